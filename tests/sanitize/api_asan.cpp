// Drives every entry point of the C ABI with arguments its host-side checks
// must reject (NULL pointers, bad sizes, misaligned pointers, unknown enums)
// and with well-formed ones, in a build of the library's host code under
// AddressSanitizer / UndefinedBehaviorSanitizer (the API layer and the MXFP4
// unit, whose host code derives the scale-factor threshold; the other
// kernel launchers are stubs that fail the run if reached).  Without a
// usable gfx950 device every well-formed call must stop at the device gate.  The host-only
// helpers (sizes, the MXFP4 scale-factor threshold) are checked for values.
// Prints "ok".
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../../include/mxq.h"
#include "../../moe_grouped_gemm_mxq_amd/csrc/mxq_internal.h"

namespace mxq {
static void reached(const char* what) {
  std::fprintf(stderr, "kernel launcher %s reached without a device\n", what);
  std::exit(3);
}
hipError_t launch_quant_row(const uint16_t*, int64_t, int64_t, int64_t, uint8_t*, uint8_t*, hipStream_t, int,
                            BatchStrides) { reached("quant_row"); return hipSuccess; }
hipError_t launch_quant_tile(const uint16_t*, int64_t, int64_t, int64_t, const int32_t*, int32_t, int64_t,
                             uint8_t*, uint8_t*, uint8_t*, uint8_t*, hipStream_t, int, BatchStrides) {
  reached("quant_tile"); return hipSuccess;
}
hipError_t launch_gemm(int, bool, const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*, float*, int64_t,
                       int64_t, int64_t, int64_t, const int32_t*, int32_t, hipStream_t) {
  reached("gemm"); return hipSuccess;
}
}  // namespace mxq

static int fails = 0;
#define EXPECT(call, want)                                                                      \
  do {                                                                                          \
    mxq_status _s = (call);                                                                     \
    if (_s != (want)) {                                                                         \
      std::fprintf(stderr, "line %d: %s gave %d, want %d (%s)\n", __LINE__, #call, (int)_s, (int)(want), \
                   mxq_last_error());                                                           \
      fails++;                                                                                  \
    } else if (_s != MXQ_OK && std::strlen(mxq_last_error()) == 0) {                            \
      std::fprintf(stderr, "line %d: no error message\n", __LINE__);                            \
      fails++;                                                                                  \
    }                                                                                           \
  } while (0)

int main() {
  alignas(256) static uint8_t buf[1 << 16];
  uint8_t* p = buf;                         // 256-byte aligned stand-in pointers (never dereferenced)
  uint16_t* x16 = reinterpret_cast<uint16_t*>(buf);
  float* f32 = reinterpret_cast<float*>(buf);
  int32_t* ge = reinterpret_cast<int32_t*>(buf);
  const mxq_status INV = MXQ_ERR_INVALID_ARGUMENT, DEV = MXQ_ERR_DEVICE, UNS = MXQ_ERR_UNSUPPORTED;

  if (mxq_abi_version() != MXQ_ABI_VERSION) fails++;
  EXPECT(mxq_device_check(-1), DEV);
  EXPECT(mxq_device_check(1 << 20), DEV);
  // host-only helpers
  int64_t cb = 0, sb = 0;
  EXPECT(mxq_operand_sizes(300, 100, MXQ_FMT_E4M3, &cb, &sb), MXQ_OK);
  if (cb != 300 * 128 || sb != 384 * 4) fails++;
  EXPECT(mxq_operand_sizes(5, 64, MXQ_FMT_E2M1, &cb, &sb), MXQ_OK);
  if (cb != 5 * 32 || sb != 128 * 2) fails++;
  EXPECT(mxq_operand_sizes(0, 64, MXQ_FMT_E4M3, &cb, &sb), INV);
  EXPECT(mxq_operand_sizes(5, 64, 7, &cb, &sb), INV);
  EXPECT(mxq_operand_sizes(5, 64, MXQ_FMT_E4M3, nullptr, &sb), INV);
  if (mxq_grouped_cols_max(100, 3) != 256 || mxq_grouped_cols_max(300, 3) != 768 || mxq_grouped_cols_max(-1, 3) != 0) fails++;
  int32_t F = 0;
  uint32_t T = 0;
  EXPECT(mxq_fp4_scale_threshold(6.0f, &F, &T), MXQ_OK);
  if (F != 3 || T != 0x7C3B7u) fails++;
  EXPECT(mxq_fp4_scale_threshold(0.0f, &F, &T), INV);
  EXPECT(mxq_fp4_scale_threshold(1e30f, &F, &T), INV);
  EXPECT(mxq_fp4_scale_threshold(6.0f, nullptr, &T), INV);
  // quantisers
  EXPECT(mxq_quantize(nullptr, 4, 4, 4, 1, p, p, nullptr, nullptr, nullptr), INV);
  EXPECT(mxq_quantize(x16, 0, 4, 4, 1, p, p, nullptr, nullptr, nullptr), INV);
  EXPECT(mxq_quantize(x16, 4, 8, 4, 1, p, p, nullptr, nullptr, nullptr), INV);
  EXPECT(mxq_quantize(x16, 4, 4, 4, 0, p, p, p, p, nullptr), INV);
  EXPECT(mxq_quantize(x16, 4, 4, 4, 4, p, p, p, p, nullptr), INV);
  EXPECT(mxq_quantize(x16, 4, 4, 4, 3, p, p, nullptr, p, nullptr), INV);
  EXPECT(mxq_quantize(x16, 4, 4, 4, 1, p + 1, p, nullptr, nullptr, nullptr), INV);
  EXPECT(mxq_quantize(x16 + 0, 4, 4, 4, 1, p, p + 2, nullptr, nullptr, nullptr), INV);
  EXPECT(mxq_quantize(reinterpret_cast<uint16_t*>(p + 1), 4, 4, 4, 1, p, p, nullptr, nullptr, nullptr), INV);
  EXPECT(mxq_quantize(x16, 4, 4, 4, 3, p, p, p, p, nullptr), DEV);
  EXPECT(mxq_quantize_batched(x16, 0, 4, 4, 4, 16, 1, p, p, nullptr, nullptr, nullptr), INV);
  EXPECT(mxq_quantize_batched(x16, 70000, 4, 4, 4, 16, 1, p, p, nullptr, nullptr, nullptr), INV);
  EXPECT(mxq_quantize_batched(x16, 2, 4, 4, 4, 3, 1, p, p, nullptr, nullptr, nullptr), INV);
  EXPECT(mxq_quantize_batched(x16, 2, 4, 4, 4, 16, 3, p, p, p, p, nullptr), DEV);
  EXPECT(mxq_quantize_grouped(x16, 64, 4, 4, nullptr, 2, 192, 2, nullptr, nullptr, p, p, nullptr), INV);
  EXPECT(mxq_quantize_grouped(x16, 64, 4, 4, ge, 0, 192, 2, nullptr, nullptr, p, p, nullptr), INV);
  EXPECT(mxq_quantize_grouped(x16, 64, 4, 4, ge, 1025, 192, 2, nullptr, nullptr, p, p, nullptr), INV);
  EXPECT(mxq_quantize_grouped(x16, 64, 4, 4, ge, 2, 100, 2, nullptr, nullptr, p, p, nullptr), INV);
  EXPECT(mxq_quantize_grouped(x16, (int64_t)1 << 32, 4, 4, ge, 2, 192, 2, nullptr, nullptr, p, p, nullptr), INV);
  EXPECT(mxq_quantize_grouped(x16, 64, 4, 4, ge, 2, 192, 3, p, p, p, p, nullptr), DEV);
  // MXFP4
  EXPECT(mxq_qdq_fp4(nullptr, f32, 2, 33, nullptr, nullptr, nullptr), INV);
  EXPECT(mxq_qdq_fp4(f32, f32, 2, 0, nullptr, nullptr, nullptr), INV);
  EXPECT(mxq_qdq_fp4(f32, f32, 2, 33, p + 1, nullptr, nullptr), INV);
  EXPECT(mxq_qdq_fp4(f32, f32, 2, 33, p, p, nullptr), DEV);
  EXPECT(mxq_qdq_fp4_ex(f32, f32, 2, 33, -6.0f, nullptr, nullptr, nullptr, nullptr), INV);
  EXPECT(mxq_qdq_fp4_ex(f32, f32, 2, 33, 6.0f, nullptr, nullptr, p + 1, nullptr), INV);
  EXPECT(mxq_qdq_fp4_ex(f32, f32, 2, 33, 5.0f, p, p, p, nullptr), DEV);
  EXPECT(mxq_quantize_fp4(f32, 2, 33, 6.0f, nullptr, p, nullptr), INV);
  EXPECT(mxq_quantize_fp4(f32, 2, 33, 1e-30f, p, p, nullptr), INV);
  EXPECT(mxq_quantize_fp4(f32, 2, 33, 6.0f, p, p, nullptr), DEV);
  EXPECT(mxq_quantize_fp4_grouped(nullptr, 64, 8, 8, ge, 2, 128, 6.0f, p, p, nullptr), INV);
  EXPECT(mxq_quantize_fp4_grouped(f32, 64, 8, 8, ge, 2, 100, 6.0f, p, p, nullptr), INV);
  EXPECT(mxq_quantize_fp4_grouped(f32, 64, 8, 8, ge, 2, 128, 6.0f, p + 8, p, nullptr), INV);
  EXPECT(mxq_quantize_fp4_grouped(f32, 64, 8, 8, ge, 2, 128, -1.0f, p, p, nullptr), INV);
  EXPECT(mxq_quantize_fp4_grouped(f32, (int64_t)1 << 31, 8, 8, ge, 2, 128, 6.0f, p, p, nullptr), INV);
  EXPECT(mxq_quantize_fp4_grouped(f32, 64, 8, 8, ge, 2, 128, 6.0f, p, p, nullptr), DEV);
  EXPECT(mxq_ste_backward_fp4(f32, p, f32 + 1, 2, 33, nullptr), INV);
  EXPECT(mxq_ste_backward_fp4(f32, p, f32, 2, 33, nullptr), DEV);
  // GEMMs
  EXPECT(mxq_gemm(p, p, p, p, f32, 4, 4, 33, 4, MXQ_FMT_E4M3, nullptr), INV);
  EXPECT(mxq_gemm(p, p, p, p, f32, 4, 4, 32, 3, MXQ_FMT_E4M3, nullptr), INV);
  EXPECT(mxq_gemm(p, p + 2, p, p, f32, 4, 4, 32, 4, MXQ_FMT_E4M3, nullptr), INV);
  EXPECT(mxq_gemm(p + 8, p, p, p, f32, 4, 4, 32, 4, MXQ_FMT_E4M3, nullptr), INV);
  EXPECT(mxq_gemm(p, p, p, p, f32, 4, 4, 32, 4, (mxq_fmt)9, nullptr), UNS);
  EXPECT(mxq_gemm(p, p, p, p, f32, 4, 4, 32, 4, MXQ_FMT_E4M3, nullptr), DEV);
  EXPECT(mxq_grouped_gemm((mxq_gg_mode)5, p, p, p, p, f32, 4, 4, 32, ge, 2, MXQ_FMT_E4M3, nullptr), INV);
  EXPECT(mxq_grouped_gemm(MXQ_GG_RAGGED_M, p, p, p, p, f32, 4, 4, 32, ge, 0, MXQ_FMT_E4M3, nullptr), INV);
  EXPECT(mxq_grouped_gemm(MXQ_GG_RAGGED_M, p, p, p, p, f32, (int64_t)1 << 32, 4, 32, ge, 2, MXQ_FMT_E4M3,
                          nullptr), INV);
  EXPECT(mxq_grouped_gemm(MXQ_GG_RAGGED_M, p, p, p, p, f32, 4, 4, 32, nullptr, 2, MXQ_FMT_E4M3, nullptr), INV);
  EXPECT(mxq_grouped_gemm(MXQ_GG_RAGGED_K, p, p, p, p, f32, 4, 4, 32, ge, 2, MXQ_FMT_E4M3, nullptr), DEV);
  EXPECT(mxq_grouped_gemm(MXQ_GG_RAGGED_M, p, p, p, p, f32, 4, 4, 32, ge, 2, MXQ_FMT_E2M1, nullptr), DEV);
  EXPECT(mxq_grouped_gemm(MXQ_GG_RAGGED_K, p, p, p, p, f32, 4, 4, 32, ge, 2, MXQ_FMT_E2M1, nullptr), DEV);
  EXPECT(mxq_validate_group_end(ge, 0, 10, ge, nullptr), INV);
  EXPECT(mxq_validate_group_end(ge, 2, -1, ge, nullptr), INV);
  EXPECT(mxq_validate_group_end(ge, 2, 10, ge, nullptr), DEV);
  if (fails) {
    std::fprintf(stderr, "%d checks failed\n", fails);
    return 1;
  }
  std::printf("ok\n");
  return 0;
}
