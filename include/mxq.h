/*
 * mxq.h -- C ABI of libmxq: MX microscaling quantisation and block-scaled
 * GEMMs for AMD Instinct MI355X (gfx950).
 *
 * The operations follow these web pages:
 *  - torchtitan-npu feature guide "低精度训练特性（MXFP8 / HiFloat8）",
 *    sections "线性层低精度" (MXFP8 linear: per-block quantisation with 32
 *    elements sharing one scale, forward, input-gradient and weight-gradient
 *    GEMMs in FP8, output returned at higher precision) and "MoE 专家层低精度"
 *    (grouped expert GEMMs; grouped per-block quantisation of the
 *    weight-gradient operands).
 *  - MindSpeed pull request 3852 (--fp8-quant-fb-split), "主要改动": expert
 *    weights quantised on both axes at once in the forward pass, or on the
 *    forward reduction axis only with the backward axis re-quantised later.
 *  - "AMCT FakeQuant 模拟伪量化工具包：MXFP4 推理精度验证与 QAT 训练实践",
 *    section 2 "MXFP4 数值模型" and section 3.3 (MXFP4 quant-dequant).
 * The pages leave the MXFP8 shared-exponent rule open; the library uses the
 * OCP MX v1.0 rule (shared = floor(log2(amax)) - 8, elements rounded to
 * nearest-even and saturated at +-448, all-zero block -> scale byte 0).
 *
 * Conventions shared by every entry point
 *  - Tensors are row-major and live in device memory of the current HIP
 *    device; host pointers are never accepted for tensor arguments.
 *  - Ownership: the caller allocates and frees every buffer.  The library
 *    never allocates or frees device memory, never synchronises, never copies
 *    group sizes back to the host and keeps no per-call state; it only caches
 *    the per-device architecture check and a thread-local error message.
 *  - Work is enqueued on the caller's stream `st` (0 = the null stream) as
 *    kernel launches only (no memset, copy or synchronisation), so a
 *    sequence of calls can be recorded into a HIP graph and replayed.
 *    Outputs must not alias inputs.  Code arrays (quantiser outputs, GEMM
 *    operands) must be 16-byte aligned; each entry point states what it
 *    requires of its other pointers (bf16 inputs 2 bytes, fp32 data and
 *    packed scale arrays that are written as dwords 4 bytes) and rejects a
 *    pointer that breaks it with MXQ_ERR_INVALID_ARGUMENT.
 *  - A quantised MXFP8 operand is `codes[rows][Kp]` (one E4M3 byte per
 *    element, the reduction axis K contiguous, Kp = ceil32(K), padding codes
 *    0x00) plus its scales: one E8M0 byte (value 2^(byte-127)) per row and
 *    block of 32, in 128-row groups -- the scale of row r, block b is byte
 *    (((r/128) * (Kp/32) + b) * 32 + r%32) * 4 + (r/32)%4 of an array of
 *    ceil128(rows) * (Kp/32) bytes ("scales[ceil128(rows)/128][Kp/32][32][4]").
 *    A dword holds the scales of rows r, r+32, r+64, r+96 of a group for one
 *    block, and a group's blocks are 128 bytes apart, which is how a GEMM
 *    tile fetches them.  Bytes of rows past `rows` are not written.  A row
 *    range whose first row is a multiple of 128 is itself a valid operand
 *    (its scale array starts at byte first_row * (Kp/32)).
 *  - "row" copy: blocks along the contiguous dim of the input.  "colT" copy:
 *    the quantised transpose, blocks running down the columns of the input.
 *  - Errors: every entry point validates its host-visible arguments first
 *    and returns a status (never aborts); on failure `mxq_last_error()`
 *    describes it.  Faults inside kernels surface at the caller's next
 *    synchronisation of the stream.  Group ends live on the device and are a
 *    precondition (non-decreasing, last <= rows); kernels clamp them so that a
 *    malformed array never makes them access memory out of bounds, and
 *    `mxq_validate_group_end` checks them on the device.
 */
#ifndef MXQ_H
#define MXQ_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MXQ_ABI_VERSION 7
#define MXQ_BLOCK 32          /* elements per MX block; fixed */
#define MXQ_MAX_GROUPS 1024   /* largest G the grouped entry points accept */
/* E4M3 GEMM reductions of at most this many elements (dense and ragged M: K;
 * ragged K: an expert's token count) run with exact 8-product MFMA groups;
 * see mxq_gemm. */
#define MXQ_EXACT_GROUPS_MAX_K 1024
/* Code bytes per operand row the GEMMs address (K for E4M3, K/2 for E2M1)
 * must stay below this: a 256-row tile of codes is addressed with 32-bit
 * offsets.  So K <= 2^23 - 32 (E4M3) and K <= 2^24 - 32 (E2M1). */
#define MXQ_GEMM_MAX_ROW_BYTES (1 << 23)

typedef enum {
    MXQ_OK = 0,
    MXQ_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, misaligned pointer, bad enum */
    MXQ_ERR_UNSUPPORTED = 2,      /* valid request the library does not implement */
    MXQ_ERR_DEVICE = 3,           /* no HIP device, or the current device is not gfx950 */
    MXQ_ERR_LAUNCH = 4,           /* the HIP runtime rejected a kernel launch */
    MXQ_STATUS_MAX_ENUM = 0x7FFFFFFF
} mxq_status;

/* Every enum of this header spans the int32 range (its *_MAX_ENUM member), so
 * a caller passing any int32 value (for instance through a foreign-function
 * binding) passes a valid value of the type; values outside the listed ones
 * are rejected with MXQ_ERR_INVALID_ARGUMENT or MXQ_ERR_UNSUPPORTED. */

/* axis bitmask for the quantisers; ROW|COLT is the dual-axis quantisation
 * (both copies from one read of the input). */
enum { MXQ_AXIS_ROW = 1, MXQ_AXIS_COLT = 2 };

/* element format of a GEMM operand: E4M3 codes (one byte each, written by
 * the MXFP8 quantisers) or E2M1 codes (two per byte, element 2j in the low
 * nibble of byte j, written by mxq_quantize_fp4) */
typedef enum { MXQ_FMT_E4M3 = 0, MXQ_FMT_E2M1 = 1, MXQ_FMT_MAX_ENUM = 0x7FFFFFFF } mxq_fmt;

/* grouped GEMM modes */
typedef enum {
    MXQ_GG_RAGGED_M = 0, /* expert forward / input gradient: rows split into groups */
    MXQ_GG_RAGGED_K = 1, /* expert weight gradient: reduction axis split into groups */
    MXQ_GG_MAX_ENUM = 0x7FFFFFFF
} mxq_gg_mode;

/* Version of this ABI (MXQ_ABI_VERSION of the built library). */
int mxq_abi_version(void);

/* Message for the last failed call on this thread ("" if none). Owned by the
 * library; valid until the next call on the same thread. */
const char* mxq_last_error(void);

/* MXQ_OK iff HIP device `device` exists and is gfx950. */
mxq_status mxq_device_check(int device);

/* Row pitch (ldq) for a grouped token-axis copy of T rows in G groups: at
 * least T + 31 G, an upper bound of sum_g ceil32(m_g), rounded up to an odd
 * multiple of 256.  Rows then start on 128-byte lines (E4M3 rows of ldq
 * bytes, E2M1 rows of ldq/2), which the weight-gradient GEMM loads whole,
 * and consecutive rows do not fall in the same memory channels (a pitch of
 * 2^10 x 129 bytes measured 1.2x slower).  Any ldq that is a multiple of 32
 * and at least sum_g ceil32(m_g) stays valid.  Pure host arithmetic. */
int64_t mxq_grouped_cols_max(int64_t T, int32_t G);

/* Bytes of a quantised GEMM operand of `rows` rows and reduction length K in
 * format fmt (MXQ_FMT_E4M3 or MXQ_FMT_E2M1), Kp = ceil32(K): *code_bytes =
 * rows * Kp (E4M3) or rows * Kp / 2 (E2M1); *scale_bytes = ceil128(rows) *
 * Kp / 32 (the operand scale layout below).  The row copy of an R x C matrix
 * is (R, C), its colT copy (C, R), a grouped token-axis copy (C, ldq), an
 * MXFP4 operand (rows, L).  The shape-only counterpart of the quantisers, so
 * a caller can allocate their outputs.  Pure host arithmetic; rows, K >= 1,
 * outputs non-NULL, else MXQ_ERR_INVALID_ARGUMENT. */
mxq_status mxq_operand_sizes(int64_t rows, int64_t K, int fmt, int64_t* code_bytes, int64_t* scale_bytes);

/*
 * MXFP8 quantisation of a bf16 matrix x [R][ldx] (R x C used), the per-block
 * quantisation of activations and weights of the torchtitan-npu guide
 * ("线性层低精度"), with the axis choice of MindSpeed PR 3852 ("主要改动").
 *   axis_mask & MXQ_AXIS_ROW : q_row [R][Cp], s_row (R rows, Cp/32 blocks,
 *                              operand layout), Cp = ceil32(C)
 *   axis_mask & MXQ_AXIS_COLT: q_colT [C][Rp], s_colT (C rows, Rp/32 blocks,
 *                              operand layout), Rp = ceil32(R)
 * Pointers for an axis not requested may be NULL.  Both axes together read
 * x once (dual-axis quantisation).  R, C >= 1; ldx >= C.  x 2-byte aligned
 * (16-byte alignment with ldx % 8 == 0 takes the vector load path), q_row
 * and q_colT 16-byte, s_row 4-byte aligned; s_colT any alignment.
 */
mxq_status mxq_quantize(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, int axis_mask,
                        uint8_t* q_row, uint8_t* s_row, uint8_t* q_colT, uint8_t* s_colT,
                        hipStream_t st);

/*
 * mxq_quantize over `batch` matrices in one launch: matrix b is
 * x + b * x_stride (bf16 elements), each [R][ldx] (R x C used) -- the
 * per-expert weights [G][K][N] of the MoE layer (torchtitan-npu guide,
 * "MoE 专家层低精度"; MindSpeed PR 3852, "主要改动").  The outputs of
 * matrix b are exactly what mxq_quantize writes for it, back to back:
 * q_row + b*R*Cp, s_row + b*ceil128(R)*(Cp/32), q_colT + b*C*Rp,
 * s_colT + b*ceil128(C)*(Rp/32) (each scale array the full operand scale
 * layout of its matrix).  1 <= batch <= 65535;
 * x_stride >= (R-1)*ldx + C when batch > 1.
 */
mxq_status mxq_quantize_batched(const uint16_t* x, int64_t batch, int64_t R, int64_t C, int64_t ldx,
                                int64_t x_stride, int axis_mask, uint8_t* q_row, uint8_t* s_row,
                                uint8_t* q_colT, uint8_t* s_colT, hipStream_t st);

/*
 * Grouped token-axis MXFP8 quantisation for the expert weight gradient
 * (torchtitan-npu guide, "MoE 专家层低精度").  x bf16 [T][ldx] (T x C used);
 * group g owns rows [end_{g-1}, end_g) with end_g = group_end[g] (device
 * int32 [G], cumulative, end_{-1} = 0).
 *   MXQ_AXIS_COLT: q_colT [C][ldq], s_colT (C rows, ldq/32 blocks,
 *     operand layout).  Blocks restart at
 *     each group start; group g occupies columns [P_g, P_g + ceil32(m_g)),
 *     P_g = sum_{j<g} ceil32(m_j), its tail zero-padded.  Columns at and past
 *     P_G are not written.  ldq % 32 == 0; ldq >= sum_g ceil32(m_g) is a
 *     precondition (mxq_grouped_cols_max(T, G) always suffices); blocks that
 *     would fall past ldq are dropped.
 *   MXQ_AXIS_ROW: q_row [T][Cp], s_row (T rows, operand layout), identical to
 *     mxq_quantize's row copy; with COLT the input is read once.
 * 1 <= G <= MXQ_MAX_GROUPS; T, C >= 1.
 */
mxq_status mxq_quantize_grouped(const uint16_t* x, int64_t T, int64_t C, int64_t ldx,
                                const int32_t* group_end, int32_t G, int64_t ldq, int axis_mask,
                                uint8_t* q_row, uint8_t* s_row, uint8_t* q_colT, uint8_t* s_colT,
                                hipStream_t st);

/*
 * MXFP4 quantise-dequantise of the AMCT FakeQuant article (section 2 and
 * section 3.3).  x, y fp32 [rows][L], L = last dim of the caller's tensor.
 * Each row is zero-padded to Lp = ceil32(L) on its own, so rows never share a
 * block.  Per block: scale = 2^round(log2(max|x|/6)) with the raw scale
 * max|x|/6 clamped at 2^-30 (round taken exactly); each element becomes the
 * E2M1 codebook value {0,0.5,1,1.5,2,3,4,6} nearest to |x|/scale, ties to the
 * larger magnitude, everything from 5 up saturating to 6; y = sign(x) * code
 * * scale (the sign of x is kept also when the code is 0).
 * Optional outputs (NULL to skip): codes [rows][Lp/2] E2M1 nibbles, element
 * 2j in the low nibble of byte j, nibble = sign<<3 | codebook index (the OCP
 * E2M1 bit pattern); scales [rows][Lp/32] E8M0 bytes, row-major (these are
 * not GEMM operands).  NaN/Inf inputs are outside the contract.  rows, L >= 1.
 */
mxq_status mxq_qdq_fp4(const float* x, float* y, int64_t rows, int64_t L,
                       uint8_t* codes, uint8_t* scales, hipStream_t st);

/*
 * MXFP4 quantise-dequantise with a runtime scale factor and the clipped-STE
 * saturation mask (AMCT FakeQuant article: scale_factor among the section 2
 * parameters, passed to the op as 6 / scale_factor in section 3.3; the
 * clipped straight-through estimator of section 4.1).  As mxq_qdq_fp4, with
 * scale = 2^round(log2(max|x| / scale_factor)) (raw scale clamped at 2^-30,
 * round taken exactly); scale_factor = 6 gives mxq_qdq_fp4's results.
 * scale_factor must be a normal fp32 value in [2^-64, 2^64), else
 * MXQ_ERR_INVALID_ARGUMENT.  Blocks whose scale would exceed 2^127, or whose
 * dequantised values overflow fp32, are outside the contract (only possible
 * for scale_factor < 6 and inputs near the fp32 maximum).
 * sat_mask (optional, NULL to skip; 4-byte aligned): device bytes
 * [rows][Lp/8]; bit j of byte k is element 8k + j of the row, set iff
 * |x| > 6 * scale (the element was clipped to the largest code); bits of the
 * padding past L are 0.  codes and scales as for mxq_qdq_fp4.
 */
mxq_status mxq_qdq_fp4_ex(const float* x, float* y, int64_t rows, int64_t L, float scale_factor,
                          uint8_t* codes, uint8_t* scales, uint8_t* sat_mask, hipStream_t st);

/*
 * Clipped-STE backward of the MXFP4 quantiser (AMCT FakeQuant article,
 * section 4.1): grad_x = 0 where the forward clipped the element (its
 * sat_mask bit, as written by mxq_qdq_fp4_ex for the same rows and L, is
 * set), grad_x = grad_y elsewhere.  grad_y, grad_x fp32 [rows][L] on the
 * device; grad_x may be grad_y (in place) but must not partly overlap it.
 * All three pointers 4-byte aligned; rows, L >= 1.
 */
mxq_status mxq_ste_backward_fp4(const float* grad_y, const uint8_t* sat_mask, float* grad_x,
                                int64_t rows, int64_t L, hipStream_t st);

/*
 * Host only (no device needed): the exponent threshold mxq_qdq_fp4_ex uses
 * for a scale factor.  With scale_factor * sqrt(2) = (1 + t) * 2^F, a block's
 * exponent is E - F + (m >= T) for max|x| = (1 + m / 2^23) * 2^E, where
 * T = ceil(t * 2^23) (T = 2^23: never).  Writes F and T; rejects factors
 * outside [2^-64, 2^64) with MXQ_ERR_INVALID_ARGUMENT.
 */
mxq_status mxq_fp4_scale_threshold(float scale_factor, int32_t* F, uint32_t* T);

/*
 * MXFP4 GEMM operand quantisation: the same block rule and element rounding
 * as mxq_qdq_fp4_ex (AMCT FakeQuant article, section 2; scale_factor 6 is the
 * default) without the dequantised output, with the scales in the layout
 * the GEMMs read.  x fp32 [rows][L] device, 4-byte aligned; each row zero-
 * padded to Lp = ceil32(L).  codes: device bytes [rows][Lp/2], 16-byte
 * aligned, E2M1 nibbles as for mxq_qdq_fp4 (element 2j in the low nibble of
 * byte j).  scales: E8M0 bytes in the GEMM operand layout of the MXFP8
 * quantisers (row r, block b at byte (((r/128)*(Lp/32) + b)*32 + r%32)*4 +
 * (r/32)%4 of a ceil128(rows)*(Lp/32)-byte array; bytes of rows past `rows`
 * are not written).  A GEMM operand with K = Lp.  scale_factor as for
 * mxq_qdq_fp4_ex.  rows, L >= 1.
 */
mxq_status mxq_quantize_fp4(const float* x, int64_t rows, int64_t L, float scale_factor, uint8_t* codes,
                            uint8_t* scales, hipStream_t st);

/*
 * Grouped token-axis MXFP4 GEMM operands for the expert weight gradient (the
 * optional MXFP4 of routed experts, torchao_npu RFC section 3.4, with the
 * numeric model of the AMCT FakeQuant article, section 2): x fp32 [T][ldx]
 * (T x C used) on the device, 4-byte aligned; group_end as for
 * mxq_quantize_grouped.  Blocks of 32 run down the token axis within each
 * group and restart at each group start; group g occupies padded positions
 * [P_g, P_g + ceil32(m_g)), P_g = sum_{j<g} ceil32(m_j), its tail zero.  The
 * block rule and element rounding are mxq_quantize_fp4's (scale_factor 6 by
 * default, same range).  codes: device bytes [C][ldq/2], 16-byte aligned,
 * E2M1 nibbles with position 2j in the low nibble of byte j; scales: E8M0
 * bytes in the GEMM operand layout (C rows, ldq/32 blocks).  Positions at
 * and past P_G are not written.  ldq % 32 == 0; ldq >= sum_g ceil32(m_g) is
 * a precondition (mxq_grouped_cols_max(T, G) suffices); blocks past ldq are
 * dropped.  1 <= G <= MXQ_MAX_GROUPS; T, C >= 1.  The operands of
 * mxq_grouped_gemm(MXQ_GG_RAGGED_K, .., MXQ_FMT_E2M1).
 */
mxq_status mxq_quantize_fp4_grouped(const float* x, int64_t T, int64_t C, int64_t ldx,
                                    const int32_t* group_end, int32_t G, int64_t ldq, float scale_factor,
                                    uint8_t* codes, uint8_t* scales, hipStream_t st);

/*
 * Block-scaled GEMM C[m][n] = sum_k deq(A)[m][k] * deq(B)[n][k] (the FP8
 * linear GEMMs of the torchtitan-npu guide, "线性层低精度"), fp32
 * accumulation and fp32 output.  A codes [M][K] + scales (M rows);
 * B codes [N][K] + scales (N rows), scales in the operand layout; C fp32 [M][ldc].
 * Forward Y = X W: A = row copy of X, B = colT copy of W [K][N].
 * Input gradient dX = dY W^T: A = row copy of dY, B = row copy of W.
 * Weight gradient dW = X^T dY: A = colT copy of X, B = colT copy of dY.
 * fmt MXQ_FMT_E2M1 (MXFP4 operands: the optional MXFP4 of routed experts in
 * the torchao_npu RFC's "mix" recipe, section 3.4, with the AMCT article's
 * numeric model, taken as a GEMM on the codes): A codes [M][K/2], B codes
 * [N][K/2] as written by mxq_quantize_fp4 (rows of K elements), scales in
 * the same operand layout.
 * M, N >= 1; K >= 32, K % 32 == 0; code bytes per row (K, or K/2 for
 * E2M1) below MXQ_GEMM_MAX_ROW_BYTES; ldc >= N.  A, B 16-byte aligned, sA,
 * sB and C 4-byte aligned (else MXQ_ERR_INVALID_ARGUMENT).  Unknown fmt:
 * MXQ_ERR_UNSUPPORTED.
 */
mxq_status mxq_gemm(const uint8_t* A, const uint8_t* sA, const uint8_t* B, const uint8_t* sB,
                    float* C, int64_t M, int64_t N, int64_t K, int64_t ldc, mxq_fmt fmt,
                    hipStream_t st);

/*
 * Grouped block-scaled GEMM over ragged expert groups (torchtitan-npu guide,
 * "MoE 专家层低精度"); group_end device int32 [G] as for mxq_quantize_grouped.
 *   MXQ_GG_RAGGED_M: A [M][K] (+ scales of M rows); B [G][N][K] with G
 *     scale arrays of N rows each, expert g's at byte g * ceil128(N) * (K/32);
 *     C fp32 [M][N].  Rows of group g use expert B[g]; rows at or past
 *     group_end[G-1] are not written.  K >= 32, K % 32 == 0.
 *     Expert forward: A = row copy of X, B[g] = colT copy of W[g] [K][N].
 *     Expert input gradient: A = row copy of dY, B[g] = row copy of W[g].
 *   MXQ_GG_RAGGED_K: A [M][K] and B [N][K] are grouped token-axis copies
 *     (K = their ldq); C fp32 [G][M][N] with
 *     C[g] = sum over group g's padded columns of deq(A) deq(B);
 *     an empty group gets exact zeros.  Expert weight gradient:
 *     A = grouped copy of X (M = hidden), B = grouped copy of dY (N = ffn).
 *     The kernel reads each group's rows from the 128-byte line at or below
 *     its first column and zeroes the columns before it, so the columns
 *     before P_g must hold quantised data (the earlier groups' blocks, as the
 *     grouped quantisers write them: no positions lie between groups).
 * fmt MXQ_FMT_E2M1: MXFP4 operands as for mxq_gemm (codes K/2 bytes per row,
 * expert g's B codes at byte g * N * K/2); for MXQ_GG_RAGGED_K the grouped
 * token-axis copies of mxq_quantize_fp4_grouped (K = their ldq).
 * M, N >= 1; K >= 32, K % 32 == 0; code bytes per row below
 * MXQ_GEMM_MAX_ROW_BYTES (as for mxq_gemm); 1 <= G <= MXQ_MAX_GROUPS.  A, B
 * 16-byte aligned, sA, sB and C 4-byte aligned (else
 * MXQ_ERR_INVALID_ARGUMENT).
 */
mxq_status mxq_grouped_gemm(mxq_gg_mode mode, const uint8_t* A, const uint8_t* sA,
                            const uint8_t* B, const uint8_t* sB, float* C,
                            int64_t M, int64_t N, int64_t K,
                            const int32_t* group_end, int32_t G, mxq_fmt fmt, hipStream_t st);

/*
 * Device-side check of a group_end array: writes 0 to *flag (device int32)
 * if group_end is non-decreasing, starts >= 0 and ends <= T, else 1 + the
 * index of the first offending entry.  Enqueued on `st`; read *flag after
 * synchronising.  1 <= G <= MXQ_MAX_GROUPS.
 */
mxq_status mxq_validate_group_end(const int32_t* group_end, int32_t G, int64_t T,
                                  int32_t* flag, hipStream_t st);

#ifdef __cplusplus
}
#endif

#endif /* MXQ_H */
