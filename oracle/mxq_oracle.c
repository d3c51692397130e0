/*
 * mxq_oracle.c -- plain, slow CPU oracle for MX microscaling quantisation and
 * block-scaled GEMMs.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the package smoke check and
 * the benchmark's CPU-baseline leg load this library.  It shares no code,
 * header, table or constant generator with the HIP library, and the HIP
 * library never calls it.
 *
 * Every quantity is computed element by element in fp64 (or exact integer
 * arithmetic) in the order the sources state it; OpenMP only splits
 * independent outputs across threads and never changes any result.
 *
 * Sources:
 *  [AMCT]  "AMCT FakeQuant 模拟伪量化工具包：MXFP4 推理精度验证与 QAT 训练实践"
 *          (cf-1.com news 4796826): section 2 "MXFP4 数值模型" (block of 32
 *          along the last dim, scale = 2^round(log2(max_abs/6)) with the raw
 *          scale clamped at 2^-30, codebook {0,±0.5,±1,±1.5,±2,±3,±4,±6},
 *          midpoint cascade with >=), section 3.3 (pad each row to a multiple
 *          of 32 before flattening, so rows never share a block).
 *  [TT]    torchtitan-npu guide "低精度训练特性（MXFP8 / HiFloat8）", sections
 *          "线性层低精度" and "MoE 专家层低精度": per-block MXFP8 quantisation
 *          of activations and weights with 32 elements sharing one scale;
 *          forward, input-gradient and weight-gradient GEMMs in FP8; grouped
 *          per-block quantisation for the expert weight gradient.
 *  [MS]    MindSpeed pull request 3852 (--fp8-quant-fb-split), "主要改动": the
 *          forward quantises expert weights on axis -2 (the forward reduction
 *          axis), the backward on axis -1.
 *  [OCP]   OCP Microscaling Formats (MX) specification v1.0, section 6.3 and
 *          the E4M3 element definition.  The pages leave the MXFP8 shared
 *          exponent rule open; this oracle takes the OCP rule
 *          shared = floor(log2(amax)) - emax(E4M3)=8, with elements rounded
 *          to nearest-even and saturated at +-448.
 *
 * Conventions: matrices are row-major; "colT" means the quantised copy of the
 * transpose, blocks running down a column of the input.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define MX_BLOCK 32

/* ---------------------------------------------------------------------- */
/* small helpers                                                           */
/* ---------------------------------------------------------------------- */

static int64_t ceil32(int64_t v) { return (v + MX_BLOCK - 1) / MX_BLOCK * MX_BLOCK; }

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads of the parallel loops that follow (n >= 1); only the timing of the
 * oracle uses it, never its results, which do not depend on the split. */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* NaN and Inf (exponent field all ones) are outside the method's contract */
static int bf16_all_finite(const uint16_t* x, int64_t R, int64_t C, int64_t ldx)
{
    for (int64_t r = 0; r < R; r++)
        for (int64_t c = 0; c < C; c++)
            if ((x[r * ldx + c] & 0x7F80) == 0x7F80) return 0;
    return 1;
}

/* bf16 bit pattern -> its exact value */
static double bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* ---------------------------------------------------------------------- */
/* FP8 E4M3 (OCP): 1 sign, 4 exponent (bias 7), 3 mantissa bits; no inf;     */
/* S.1111.111 is NaN; largest finite magnitude 448 = 1.75 * 2^8.            */
/* ---------------------------------------------------------------------- */

double oracle_e4m3_decode(uint8_t code)
{
    int s = code >> 7, e = (code >> 3) & 0xF, m = code & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        v = m * ldexp(1.0, -9);               /* subnormal: m/8 * 2^(1-7) */
    else
        v = (1.0 + m / 8.0) * ldexp(1.0, e - 7);
    return s ? -v : v;
}

/*
 * Nearest finite E4M3 value to v, ties to the code with an even mantissa,
 * magnitudes beyond 448 saturating to 448, sign kept (also for zero).
 * Plain search over the 127 non-negative finite codes, which are ordered by
 * value: find the last code not above |v|, then compare with its successor.
 */
uint8_t oracle_e4m3_encode(double v)
{
    double a = fabs(v);
    int lo = 0, hi = 0x7E;
    uint8_t code;
    if (a >= oracle_e4m3_decode(0x7E)) {
        code = 0x7E;
    } else {
        while (hi - lo > 1) {               /* invariant: val(lo) <= a < val(hi) */
            int mid = (lo + hi) / 2;
            if (oracle_e4m3_decode((uint8_t)mid) <= a) lo = mid; else hi = mid;
        }
        double dlo = a - oracle_e4m3_decode((uint8_t)lo);
        double dhi = oracle_e4m3_decode((uint8_t)hi) - a;
        if (dlo < dhi) code = (uint8_t)lo;
        else if (dhi < dlo) code = (uint8_t)hi;
        else code = (uint8_t)((lo & 1) == 0 ? lo : hi);   /* tie: even mantissa */
    }
    if (signbit(v)) code |= 0x80;
    return code;
}

/* element-wise oracle_e4m3_encode over an array */
void oracle_e4m3_encode_n(const double* v, int64_t n, uint8_t* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) out[i] = oracle_e4m3_encode(v[i]);
}

/* E8M0 byte -> 2^(byte-127); 0xFF is NaN */
double oracle_e8m0_decode(uint8_t byte)
{
    if (byte == 0xFF) return NAN;
    return ldexp(1.0, (int)byte - 127);
}

/* ---------------------------------------------------------------------- */
/* MXFP8 quantisation of one block of (up to) 32 bf16 values [TT], [OCP]    */
/* ---------------------------------------------------------------------- */

/* shared exponent: floor(log2(amax)) - 8, clamped to the E8M0 range; an
 * all-zero block takes the smallest scale (byte 0x00). */
static int mxfp8_shared_exp(double amax)
{
    int e2;
    if (amax == 0.0) return -127;
    frexp(amax, &e2);                 /* amax = f * 2^e2, f in [0.5, 1) */
    int s = (e2 - 1) - 8;             /* floor(log2 amax) - emax(E4M3) */
    if (s < -127) s = -127;
    if (s > 127) s = 127;
    return s;
}

/* vals[0..n-1] (n <= 32, the rest of the block is zero padding) -> 32 codes
 * and one scale byte. */
static void mxfp8_block(const double* vals, int n, uint8_t* codes, uint8_t* scale)
{
    double amax = 0.0;
    for (int i = 0; i < n; i++)
        if (fabs(vals[i]) > amax) amax = fabs(vals[i]);
    int s = mxfp8_shared_exp(amax);
    *scale = (uint8_t)(s + 127);
    for (int i = 0; i < MX_BLOCK; i++) {
        double v = i < n ? vals[i] : 0.0;
        codes[i] = oracle_e4m3_encode(ldexp(v, -s));   /* exact: power-of-two shift */
    }
}

/* Row copy: blocks along the contiguous dim C.
 * x bf16 [R][ldx] (R x C used) -> q [R][Cp], s [R][Cp/32], Cp = ceil32(C). */
int oracle_mxfp8_quant_row(const uint16_t* x, int64_t R, int64_t C, int64_t ldx,
                           uint8_t* q, uint8_t* s)
{
    if (R < 0 || C < 0 || ldx < C) return 1;
    if (!bf16_all_finite(x, R, C, ldx)) return 2;
    int64_t Cp = ceil32(C), nb = Cp / MX_BLOCK;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; r++) {
        double vals[MX_BLOCK];
        for (int64_t b = 0; b < nb; b++) {
            int n = 0;
            for (int i = 0; i < MX_BLOCK && b * MX_BLOCK + i < C; i++, n++)
                vals[i] = bf16_value(x[r * ldx + b * MX_BLOCK + i]);
            mxfp8_block(vals, n, q + r * Cp + b * MX_BLOCK, s + r * nb + b);
        }
    }
    return 0;
}

/* Column copy (quantised transpose): blocks run down each column.
 * x bf16 [R][ldx] -> q [C][Rp], s [C][Rp/32], Rp = ceil32(R). */
int oracle_mxfp8_quant_colT(const uint16_t* x, int64_t R, int64_t C, int64_t ldx,
                            uint8_t* q, uint8_t* s)
{
    if (R < 0 || C < 0 || ldx < C) return 1;
    if (!bf16_all_finite(x, R, C, ldx)) return 2;
    int64_t Rp = ceil32(R), nb = Rp / MX_BLOCK;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < C; c++) {
        double vals[MX_BLOCK];
        for (int64_t b = 0; b < nb; b++) {
            int n = 0;
            for (int i = 0; i < MX_BLOCK && b * MX_BLOCK + i < R; i++, n++)
                vals[i] = bf16_value(x[(b * MX_BLOCK + i) * ldx + c]);
            mxfp8_block(vals, n, q + c * Rp + b * MX_BLOCK, s + c * nb + b);
        }
    }
    return 0;
}

/* Grouped token-axis column copy for the expert weight gradient [TT]:
 * group g owns rows [start_g, end_g) with end_g = group_end[g] and
 * start_g = end_{g-1} (start_0 = 0).  Blocks restart at every group start and
 * the group's tail is zero-padded, so groups never share a block.  Group g's
 * tokens occupy output columns [P_g, P_g + ceil32(m_g)),
 * P_g = sum_{j<g} ceil32(m_j).  q [C][ldq], s [C][ldq/32]; columns at and
 * beyond P_G are left untouched.  Returns nonzero on malformed group ends. */
int oracle_mxfp8_quant_grouped_colT(const uint16_t* x, int64_t T, int64_t C, int64_t ldx,
                                    const int32_t* group_end, int32_t G, int64_t ldq,
                                    uint8_t* q, uint8_t* s)
{
    if (T < 0 || C < 0 || ldx < C || G < 0 || ldq % MX_BLOCK) return 1;
    if (!bf16_all_finite(x, T, C, ldx)) return 2;
    int64_t prev = 0, need = 0;
    for (int32_t g = 0; g < G; g++) {
        if (group_end[g] < prev || group_end[g] > T) return 2;
        need += ceil32(group_end[g] - prev);
        prev = group_end[g];
    }
    if (need > ldq) return 3;
    int64_t ldsc = ldq / MX_BLOCK;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < C; c++) {
        double vals[MX_BLOCK];
        int64_t start = 0, P = 0;
        for (int32_t g = 0; g < G; g++) {
            int64_t end = group_end[g], m = end - start;
            for (int64_t b = 0; b < ceil32(m) / MX_BLOCK; b++) {
                int n = 0;
                for (int i = 0; i < MX_BLOCK && b * MX_BLOCK + i < m; i++, n++)
                    vals[i] = bf16_value(x[(start + b * MX_BLOCK + i) * ldx + c]);
                mxfp8_block(vals, n, q + c * ldq + P + b * MX_BLOCK,
                            s + c * ldsc + P / MX_BLOCK + b);
            }
            P += ceil32(m);
            start = end;
        }
    }
    return 0;
}

/* Dequantise a quantised operand q [R][K], s [R][K/32] into fp64 (exact). */
void oracle_mxfp8_dequant(const uint8_t* q, const uint8_t* s, int64_t R, int64_t K, double* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; r++)
        for (int64_t k = 0; k < K; k++)
            out[r * K + k] = oracle_e4m3_decode(q[r * K + k]) *
                             oracle_e8m0_decode(s[r * (K / MX_BLOCK) + k / MX_BLOCK]);
}

/* ---------------------------------------------------------------------- */
/* MXFP4 quantise-dequantise [AMCT section 2, section 3.3]                  */
/* ---------------------------------------------------------------------- */

/* E2M1 codebook (magnitudes) and the midpoints between neighbours. */
static const double fp4_codebook[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
static const double fp4_midpoints[7] = {0.25, 0.75, 1.25, 1.75, 2.50, 3.50, 5.00};
#define FP4_SCALE_FACTOR 6.0             /* default scale_factor [AMCT section 2] */
#define FP4_CODE_MAX 6.0                 /* largest codebook magnitude */
#define FP4_MIN_SCALE_EXP (-30)          /* raw scale clamped at 2^-30 */

/* round(log2(amax / sf)) evaluated exactly.  log2 of a rational is never an
 * odd multiple of 1/2, so there is no tie and the nearest integer n is the
 * one with 2^(n-1/2) <= amax/sf < 2^(n+1/2), i.e.
 * sf^2 * 2^(2n-1) <= amax^2 < sf^2 * 2^(2n+1) (18*4^n and 72*4^n for the
 * default sf = 6).  amax and sf are fp32 values, so amax^2, sf^2 (48
 * significant bits each) and the bounds are exact in fp64; a floating-point
 * first guess is corrected by those exact comparisons. */
static int fp4_round_log2_ratio(double amax, double sf)
{
    int n = (int)floor(log2(amax / sf) + 0.5);
    double a2 = amax * amax, s2 = sf * sf;
    while (a2 >= s2 * ldexp(2.0, 2 * n)) n++;
    while (a2 < s2 * ldexp(0.5, 2 * n)) n--;
    return n;
}

/* Scale exponent of one block: raw = max(amax/sf, 2^-30), e = round(log2 raw). */
static int fp4_scale_exp(double amax, double sf)
{
    if (amax <= sf * ldexp(1.0, FP4_MIN_SCALE_EXP))
        return FP4_MIN_SCALE_EXP;                  /* clamped raw scale */
    int n = fp4_round_log2_ratio(amax, sf);
    return n < FP4_MIN_SCALE_EXP ? FP4_MIN_SCALE_EXP : n;
}

/* Element rounding: the midpoint cascade -- the code is raised to the next
 * codebook value whenever |y| >= the midpoint below it, so ties go to the
 * larger magnitude and everything from 5 upwards becomes 6. */
static int fp4_code_index(double yabs)
{
    int idx = 0;
    for (int i = 0; i < 7; i++)
        if (yabs >= fp4_midpoints[i]) idx = i + 1;
    return idx;
}

/*
 * x fp32 [rows][L] -> y fp32 [rows][L], with scale = 2^round(log2(amax /
 * scale_factor)) [AMCT section 2; the op's inv_scale_factor_scale is
 * 6 / scale_factor, section 3.3].  Each row is padded with zeros to
 * Lp = ceil32(L) before blocking, so rows never share a block.
 * Optional outputs (may be NULL): codes [rows][Lp/2] E2M1 nibbles (element 2j
 * in the low nibble of byte j, nibble = sign<<3 | codebook index, which is
 * the OCP E2M1 bit pattern), scales [rows][Lp/32] E8M0 bytes (e + 127), and
 * the clipped-STE saturation mask [rows][Lp/8] [AMCT section 4.1]: bit j of
 * byte k is set iff |x| > 6 * scale for element 8k + j (padding: clear).
 * Returns 1 for bad sizes or a scale factor that is not positive and finite,
 * 2 if an input is NaN/Inf, a block scale exceeds 2^127 (not an E8M0 value)
 * or a dequantised value does not fit in fp32 (outside the method's contract).
 */
int oracle_mxfp4_qdq_ex(const float* x, float* y, int64_t rows, int64_t L, float scale_factor_f32,
                        uint8_t* codes, uint8_t* scales, uint8_t* sat_mask)
{
    double scale_factor = (double)scale_factor_f32;   /* an fp32 value: its square is exact in fp64 */
    if (rows < 0 || L < 0 || !(scale_factor > 0.0) || !isfinite(scale_factor)) return 1;
    int64_t Lp = ceil32(L), nb = Lp / MX_BLOCK;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t b = 0; b < nb; b++) {
            double v[MX_BLOCK];
            double amax = 0.0;
            for (int i = 0; i < MX_BLOCK; i++) {
                int64_t col = b * MX_BLOCK + i;
                v[i] = col < L ? (double)x[r * L + col] : 0.0;      /* row padding */
                if (!isfinite(v[i])) bad = 1;
                if (fabs(v[i]) > amax) amax = fabs(v[i]);
            }
            if (!isfinite(amax)) { bad = 1; continue; }
            int e = fp4_scale_exp(amax, scale_factor);
            if (e > 127) { bad = 1; continue; }               /* E8M0 tops out at 2^127 (0xFF is NaN) */
            double scale = ldexp(1.0, e);
            if (scales) scales[r * nb + b] = (uint8_t)(e + 127);
            for (int i = 0; i < MX_BLOCK; i++) {
                double yabs = fabs(v[i]) / scale;                  /* exact */
                int idx = fp4_code_index(yabs);
                double out = copysign(fp4_codebook[idx] * scale, v[i]);
                int64_t col = b * MX_BLOCK + i;
                if (col < L) {
                    if (fabs(out) > 3.4028234663852886e38) bad = 1;
                    y[r * L + col] = (float)out;                   /* exact */
                }
                if (codes) {
                    uint8_t nib = (uint8_t)((signbit(v[i]) ? 8 : 0) | idx);
                    uint8_t* byte = &codes[r * (Lp / 2) + col / 2];
                    if (col % 2 == 0) *byte = (uint8_t)((*byte & 0xF0) | nib);
                    else *byte = (uint8_t)((*byte & 0x0F) | (nib << 4));
                }
                if (sat_mask) {
                    uint8_t* byte = &sat_mask[r * (Lp / 8) + col / 8];
                    uint8_t bit = (uint8_t)(1u << (col % 8));
                    if (fabs(v[i]) > FP4_CODE_MAX * scale) *byte |= bit;
                    else *byte &= (uint8_t)~bit;
                }
            }
        }
    }
    return bad ? 2 : 0;
}

int oracle_mxfp4_qdq(const float* x, float* y, int64_t rows, int64_t L,
                     uint8_t* codes, uint8_t* scales)
{
    return oracle_mxfp4_qdq_ex(x, y, rows, L, (float)FP4_SCALE_FACTOR, codes, scales, NULL);
}

/*
 * Clipped-STE backward [AMCT section 4.1]: the gradient passes straight
 * through the quantiser except where the element saturated, where it is 0:
 * grad_x = mask ? 0 : grad_y, mask as written by oracle_mxfp4_qdq_ex.
 */
void oracle_mxfp4_ste_backward(const float* grad_y, const uint8_t* sat_mask, float* grad_x,
                               int64_t rows, int64_t L)
{
    int64_t Lp = ceil32(L);
    for (int64_t r = 0; r < rows; r++)
        for (int64_t c = 0; c < L; c++) {
            int sat = (sat_mask[r * (Lp / 8) + c / 8] >> (c % 8)) & 1;
            grad_x[r * L + c] = sat ? 0.0f : grad_y[r * L + c];
        }
}

/* ---------------------------------------------------------------------- */
/* MXFP4 operands: dequantisation and the block-scaled FP4 GEMM.            */

/* OCP E2M1 element: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa;
 * exponent 0 is subnormal (0.5 * mantissa).  The eight magnitudes are the
 * AMCT article's codebook {0, 0.5, 1, 1.5, 2, 3, 4, 6} (section 2). */
static double fp4_decode(uint8_t nib)
{
    int e = (nib >> 1) & 3, m = nib & 1;
    double mag = e == 0 ? 0.5 * m : (1.0 + 0.5 * m) * ldexp(1.0, e - 1);
    return (nib & 8) ? -mag : mag;
}

/* codes [rows][Lp/2] (element 2j in the low nibble of byte j), scales
 * [rows][Lp/32] E8M0 row-major, as written by oracle_mxfp4_qdq_ex ->
 * out [rows][L] = decode(nibble) * 2^(scale - 127). */
void oracle_mxfp4_dequant(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t L, double* out)
{
    int64_t Lp = ceil32(L);
    for (int64_t r = 0; r < rows; r++)
        for (int64_t c = 0; c < L; c++) {
            uint8_t byte = codes[r * (Lp / 2) + c / 2];
            uint8_t nib = (c % 2 == 0) ? (uint8_t)(byte & 0xF) : (uint8_t)(byte >> 4);
            int s = scales[r * (Lp / MX_BLOCK) + c / MX_BLOCK];
            out[r * L + c] = fp4_decode(nib) * ldexp(1.0, s - 127);
        }
}

/* C[m][n] = sum_k deq(A)[m][k] * deq(B)[n][k] over MXFP4 operands: A codes
 * [M][K/2] + scales [M][K/32], B codes [N][K/2] + scales [N][K/32] (the
 * layout above), K % 32 == 0; fp64, with sum |products| beside it. */
int oracle_gemm_fp4(const uint8_t* A, const uint8_t* sA, const uint8_t* B, const uint8_t* sB,
                    int64_t M, int64_t N, int64_t K, double* C, double* Cabs)
{
    if (M < 0 || N < 0 || K < 0 || K % MX_BLOCK) return 1;
    double* Xa = (double*)malloc(sizeof(double) * (size_t)(M * K + 1));
    double* Xb = (double*)malloc(sizeof(double) * (size_t)(N * K + 1));
    if (!Xa || !Xb) { free(Xa); free(Xb); return 4; }
    oracle_mxfp4_dequant(A, sA, M, K, Xa);
    oracle_mxfp4_dequant(B, sB, N, K, Xb);
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++) {
            double acc = 0.0, accabs = 0.0;
            for (int64_t k = 0; k < K; k++) {
                double p = Xa[m * K + k] * Xb[n * K + k];
                acc += p;
                accabs += fabs(p);
            }
            C[m * N + n] = acc;
            Cabs[m * N + n] = accabs;
        }
    free(Xa);
    free(Xb);
    return 0;
}

/* Selected outputs (mi[i], ni[i]) of the FP4 GEMM above. */
int oracle_gemm_fp4_sampled(const uint8_t* A, const uint8_t* sA, const uint8_t* B, const uint8_t* sB,
                            int64_t M, int64_t N, int64_t K, const int64_t* mi, const int64_t* ni,
                            int64_t count, double* C, double* Cabs)
{
    if (K % MX_BLOCK) return 1;
    for (int64_t i = 0; i < count; i++)
        if (mi[i] < 0 || mi[i] >= M || ni[i] < 0 || ni[i] >= N) return 1;
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < count; i++) {
        double a[MX_BLOCK], b[MX_BLOCK], acc = 0.0, accabs = 0.0;
        for (int64_t k0 = 0; k0 < K; k0 += MX_BLOCK) {
            /* one 32-block of row mi[i] of A and row ni[i] of B */
            oracle_mxfp4_dequant(A + mi[i] * (K / 2) + k0 / 2, sA + mi[i] * (K / MX_BLOCK) + k0 / MX_BLOCK, 1,
                                 MX_BLOCK, a);
            oracle_mxfp4_dequant(B + ni[i] * (K / 2) + k0 / 2, sB + ni[i] * (K / MX_BLOCK) + k0 / MX_BLOCK, 1,
                                 MX_BLOCK, b);
            for (int j = 0; j < MX_BLOCK; j++) {
                double p = a[j] * b[j];
                acc += p;
                accabs += fabs(p);
            }
        }
        C[i] = acc;
        Cabs[i] = accabs;
    }
    return 0;
}

/* ---------------------------------------------------------------------- */
/* Block-scaled GEMMs [TT]: C[m][n] = sum_k deq(A)[m][k] * deq(B)[n][k].    */
/* Alongside each value the oracle returns sum_k |deq(A)*deq(B)|, the scale */
/* of the tolerance an fp32-accumulating kernel is held to.                 */
/* ---------------------------------------------------------------------- */

static double deq(const uint8_t* q, const uint8_t* s, int64_t row, int64_t ldq, int64_t k)
{
    return oracle_e4m3_decode(q[row * ldq + k]) *
           oracle_e8m0_decode(s[row * (ldq / MX_BLOCK) + k / MX_BLOCK]);
}

/* one output element over K range [k0, k1) of rows a_row / b_row */
static void dot_range(const uint8_t* A, const uint8_t* sA, int64_t a_row,
                      const uint8_t* B, const uint8_t* sB, int64_t b_row,
                      int64_t ld, int64_t k0, int64_t k1, double* c, double* cabs)
{
    double acc = 0.0, accabs = 0.0;
    for (int64_t k = k0; k < k1; k++) {
        double p = deq(A, sA, a_row, ld, k) * deq(B, sB, b_row, ld, k);  /* exact */
        acc += p;
        accabs += fabs(p);
    }
    *c = acc;
    *cabs = accabs;
}

/* Dense: A [M][K], B [N][K] (K % 32 == 0) -> C [M][N], Cabs [M][N]. */
int oracle_gemm(const uint8_t* A, const uint8_t* sA, const uint8_t* B, const uint8_t* sB,
                int64_t M, int64_t N, int64_t K, double* C, double* Cabs)
{
    if (M < 0 || N < 0 || K < 0 || K % MX_BLOCK) return 1;
    double* Ad = (double*)malloc(sizeof(double) * (size_t)(M * K + 1));
    double* Bd = (double*)malloc(sizeof(double) * (size_t)(N * K + 1));
    if (!Ad || !Bd) { free(Ad); free(Bd); return 4; }
    oracle_mxfp8_dequant(A, sA, M, K, Ad);
    oracle_mxfp8_dequant(B, sB, N, K, Bd);
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++) {
            double acc = 0.0, accabs = 0.0;
            for (int64_t k = 0; k < K; k++) {
                double p = Ad[m * K + k] * Bd[n * K + k];
                acc += p;
                accabs += fabs(p);
            }
            C[m * N + n] = acc;
            Cabs[m * N + n] = accabs;
        }
    free(Ad);
    free(Bd);
    return 0;
}

/* Dense, selected outputs only: (mi[i], ni[i]) for i < count. */
int oracle_gemm_sampled(const uint8_t* A, const uint8_t* sA, const uint8_t* B, const uint8_t* sB,
                        int64_t M, int64_t N, int64_t K, const int64_t* mi, const int64_t* ni,
                        int64_t count, double* C, double* Cabs)
{
    if (K % MX_BLOCK) return 1;
    for (int64_t i = 0; i < count; i++)
        if (mi[i] < 0 || mi[i] >= M || ni[i] < 0 || ni[i] >= N) return 1;
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < count; i++)
        dot_range(A, sA, mi[i], B, sB, ni[i], K, 0, K, &C[i], &Cabs[i]);
    return 0;
}

static int check_group_end(const int32_t* group_end, int32_t G, int64_t T)
{
    int64_t prev = 0;
    for (int32_t g = 0; g < G; g++) {
        if (group_end[g] < prev || group_end[g] > T) return 1;
        prev = group_end[g];
    }
    return 0;
}

/* group of row m under cumulative ends: first g with m < group_end[g]; G if none */
static int32_t group_of_row(const int32_t* group_end, int32_t G, int64_t m)
{
    for (int32_t g = 0; g < G; g++)
        if (m < group_end[g]) return g;
    return G;
}

/* Ragged M (expert forward / input gradient): rows [start_g, end_g) of
 * A [T][K] multiply expert g's B[g] [N][K]; C [T][N].  Rows that belong to no
 * group (at or beyond group_end[G-1]) are left untouched. */
int oracle_grouped_gemm_ragged_m(const uint8_t* A, const uint8_t* sA, const uint8_t* B,
                                 const uint8_t* sB, int64_t T, int64_t N, int64_t K,
                                 const int32_t* group_end, int32_t G, double* C, double* Cabs)
{
    if (K % MX_BLOCK || check_group_end(group_end, G, T)) return 1;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t m = 0; m < T; m++) {
        int32_t g = group_of_row(group_end, G, m);
        if (g == G) continue;
        const uint8_t* Bg = B + (int64_t)g * N * K;
        const uint8_t* sBg = sB + (int64_t)g * N * (K / MX_BLOCK);
        for (int64_t n = 0; n < N; n++)
            dot_range(A, sA, m, Bg, sBg, n, K, 0, K, &C[m * N + n], &Cabs[m * N + n]);
    }
    return 0;
}

int oracle_grouped_gemm_ragged_m_sampled(const uint8_t* A, const uint8_t* sA, const uint8_t* B,
                                         const uint8_t* sB, int64_t T, int64_t N, int64_t K,
                                         const int32_t* group_end, int32_t G,
                                         const int64_t* mi, const int64_t* ni, int64_t count,
                                         double* C, double* Cabs)
{
    if (K % MX_BLOCK || check_group_end(group_end, G, T)) return 1;
    for (int64_t i = 0; i < count; i++)
        if (mi[i] < 0 || mi[i] >= T || ni[i] < 0 || ni[i] >= N ||
            group_of_row(group_end, G, mi[i]) == G) return 1;
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < count; i++) {
        int32_t g = group_of_row(group_end, G, mi[i]);
        dot_range(A, sA, mi[i], B + (int64_t)g * N * K, sB + (int64_t)g * N * (K / MX_BLOCK),
                  ni[i], K, 0, K, &C[i], &Cabs[i]);
    }
    return 0;
}

/* Ragged K (expert weight gradient): A [M][ldk] and B [N][ldk] are grouped
 * token-axis column copies; group g reduces over its padded token columns
 * [P_g, P_g + ceil32(m_g)).  C [G][M][N]; an empty group yields the empty
 * sum, exact zeros. */
int oracle_grouped_gemm_ragged_k(const uint8_t* A, const uint8_t* sA, const uint8_t* B,
                                 const uint8_t* sB, int64_t M, int64_t N, int64_t ldk,
                                 const int32_t* group_end, int32_t G, double* C, double* Cabs)
{
    if (ldk % MX_BLOCK || G < 0) return 1;
    int64_t* P = (int64_t*)malloc(sizeof(int64_t) * (size_t)(G + 1));
    if (!P) return 4;
    int64_t prev = 0;
    P[0] = 0;
    for (int32_t g = 0; g < G; g++) {
        if (group_end[g] < prev) { free(P); return 1; }
        P[g + 1] = P[g] + ceil32(group_end[g] - prev);
        prev = group_end[g];
    }
    if (P[G] > ldk) { free(P); return 1; }
#pragma omp parallel for collapse(2) schedule(dynamic, 4)
    for (int32_t g = 0; g < G; g++)
        for (int64_t m = 0; m < M; m++)
            for (int64_t n = 0; n < N; n++) {
                int64_t o = ((int64_t)g * M + m) * N + n;
                dot_range(A, sA, m, B, sB, n, ldk, P[g], P[g + 1], &C[o], &Cabs[o]);
            }
    free(P);
    return 0;
}

int oracle_grouped_gemm_ragged_k_sampled(const uint8_t* A, const uint8_t* sA, const uint8_t* B,
                                         const uint8_t* sB, int64_t M, int64_t N, int64_t ldk,
                                         const int32_t* group_end, int32_t G,
                                         const int32_t* gi, const int64_t* mi, const int64_t* ni,
                                         int64_t count, double* C, double* Cabs)
{
    if (ldk % MX_BLOCK || G < 0) return 1;
    int64_t* P = (int64_t*)malloc(sizeof(int64_t) * (size_t)(G + 1));
    if (!P) return 4;
    int64_t prev = 0;
    P[0] = 0;
    for (int32_t g = 0; g < G; g++) {
        if (group_end[g] < prev) { free(P); return 1; }
        P[g + 1] = P[g] + ceil32(group_end[g] - prev);
        prev = group_end[g];
    }
    int bad = P[G] > ldk;
    for (int64_t i = 0; i < count && !bad; i++)
        bad = gi[i] < 0 || gi[i] >= G || mi[i] < 0 || mi[i] >= M || ni[i] < 0 || ni[i] >= N;
    if (bad) { free(P); return 1; }
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < count; i++)
        dot_range(A, sA, mi[i], B, sB, ni[i], ldk, P[gi[i]], P[gi[i] + 1], &C[i], &Cabs[i]);
    free(P);
    return 0;
}
