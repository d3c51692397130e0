// Host-side launchers of the libmxq kernels (arguments already validated).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxq {

// Longest reduction that the E4M3 GEMMs run with one real product per
// 8-product MFMA group (exact group sums); MXQ_EXACT_GROUPS_MAX_K of mxq.h.
constexpr int kIlvMaxK = 1024;

// number of compute units of the current device (cached per device)
int device_cu_count();

// MXFP8 row copy: x bf16 [R][ldx] -> q [R][Cp], s [R][Cp/32]
// Element (x, bf16) and byte (outputs) offsets between the matrices of a
// batch; matrix b is handled by blockIdx.y == b.
struct BatchStrides {
  int64_t x, q_row, s_row, q_colT, s_colT;
};

hipError_t launch_quant_row(const uint16_t* x, int64_t R, int64_t C, int64_t ldx,
                            uint8_t* q, uint8_t* s, hipStream_t st, int batch = 1,
                            BatchStrides bs = BatchStrides{0, 0, 0, 0, 0});

// MXFP8 column copy (and optionally the row copy from the same read).
// grouped: group_end != nullptr; colT width ldq (multiple of 32).
hipError_t launch_quant_tile(const uint16_t* x, int64_t R, int64_t C, int64_t ldx,
                             const int32_t* group_end, int32_t G, int64_t ldq,
                             uint8_t* q_row, uint8_t* s_row, uint8_t* q_colT, uint8_t* s_colT,
                             hipStream_t st, int batch = 1, BatchStrides bs = BatchStrides{0, 0, 0, 0, 0});

// MXFP4 quant-dequant.  (F, T) encode the scale factor's exponent threshold;
// fp4_scale_params computes them and rejects factors outside [2^-64, 2^64).
bool fp4_scale_params(float scale_factor, int* F, uint32_t* T);
// y may be null (quantise only); operand_layout: scales in the GEMM operand
// layout (scale_offset) instead of row-major.
hipError_t launch_qdq_fp4(const float* x, float* y, int64_t rows, int64_t L, int F, uint32_t T,
                          uint8_t* codes, uint8_t* scales, uint8_t* sat_mask, hipStream_t st,
                          bool operand_layout = false);
hipError_t launch_ste_backward_fp4(const float* grad_y, const uint8_t* sat_mask, float* grad_x,
                                   int64_t rows, int64_t L, hipStream_t st);
// MXFP4 grouped token-axis GEMM operand: x fp32 [T][ldx] -> codes [C][ldq/2],
// scales (C rows, ldq/32 blocks, operand layout); (F, Tth) as for launch_qdq_fp4.
hipError_t launch_quant_fp4_grouped(const float* x, int64_t T, int64_t C, int64_t ldx, const int32_t* group_end,
                                    int32_t G, int64_t ldq, int F, uint32_t Tth, uint8_t* codes, uint8_t* scales,
                                    hipStream_t st);

// Block-scaled GEMMs.  mode 0: dense (G = 1, no group_end); 1: ragged M; 2: ragged K.
// fp4: E2M1 codes (two per byte) instead of E4M3.
hipError_t launch_gemm(int mode, bool fp4, const uint8_t* A, const uint8_t* sA, const uint8_t* B,
                       const uint8_t* sB, float* C, int64_t M, int64_t N, int64_t K, int64_t ldc,
                       const int32_t* group_end, int32_t G, hipStream_t st);

hipError_t launch_validate_group_end(const int32_t* group_end, int32_t G, int64_t T, int32_t* flag,
                                     hipStream_t st);

}  // namespace mxq
