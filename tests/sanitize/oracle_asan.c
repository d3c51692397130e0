/* Exercises the oracle's C entry points on small and edge-case inputs so that
 * an AddressSanitizer / UndefinedBehaviorSanitizer build can watch every
 * access: quantisers (row, column, grouped with empty and ragged groups),
 * dequantisation, MXFP4 QDQ with codes, scales and mask, the clipped-STE
 * backward, and every GEMM (dense, FP4, sampled, ragged M, ragged K), plus
 * the rejected inputs (malformed group ends, bad sizes).  Prints "ok". */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_mxfp8_quant_row(const uint16_t*, int64_t, int64_t, int64_t, uint8_t*, uint8_t*);
int oracle_mxfp8_quant_colT(const uint16_t*, int64_t, int64_t, int64_t, uint8_t*, uint8_t*);
int oracle_mxfp8_quant_grouped_colT(const uint16_t*, int64_t, int64_t, int64_t, const int32_t*, int32_t,
                                    int64_t, uint8_t*, uint8_t*);
void oracle_mxfp8_dequant(const uint8_t*, const uint8_t*, int64_t, int64_t, double*);
int oracle_mxfp4_qdq_ex(const float*, float*, int64_t, int64_t, float, uint8_t*, uint8_t*, uint8_t*);
void oracle_mxfp4_ste_backward(const float*, const uint8_t*, float*, int64_t, int64_t);
void oracle_mxfp4_dequant(const uint8_t*, const uint8_t*, int64_t, int64_t, double*);
int oracle_gemm(const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*, int64_t, int64_t, int64_t,
                double*, double*);
int oracle_gemm_sampled(const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*, int64_t, int64_t,
                        int64_t, const int64_t*, const int64_t*, int64_t, double*, double*);
int oracle_gemm_fp4(const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*, int64_t, int64_t, int64_t,
                    double*, double*);
int oracle_grouped_gemm_ragged_m(const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*, int64_t,
                                 int64_t, int64_t, const int32_t*, int32_t, double*, double*);
int oracle_grouped_gemm_ragged_k(const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*, int64_t,
                                 int64_t, int64_t, const int32_t*, int32_t, double*, double*);

static uint64_t rng = 88172645463325252ull;
static uint32_t next(void) {
  rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
  return (uint32_t)rng;
}
/* a finite bf16 with a random sign, exponent field 100..140 and mantissa */
static uint16_t rand_bf16(void) {
  uint32_t r = next();
  return (uint16_t)(((r & 1u) << 15) | ((100u + (r >> 1) % 41u) << 7) | ((r >> 8) & 0x7Fu));
}
static void* xmalloc(size_t n) {
  void* p = malloc(n ? n : 1);
  if (!p) { fprintf(stderr, "out of memory\n"); exit(2); }
  memset(p, 0, n ? n : 1);
  return p;
}
#define CHECK(cond) do { if (!(cond)) { fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__); return 1; } } while (0)

static int shapes(int64_t R, int64_t C) {
  int64_t Cp = (C + 31) / 32 * 32, Rp = (R + 31) / 32 * 32;
  uint16_t* x = xmalloc(sizeof(uint16_t) * R * C);
  for (int64_t i = 0; i < R * C; i++) x[i] = rand_bf16();
  uint8_t* q = xmalloc(R * Cp); uint8_t* s = xmalloc(R * Cp / 32);
  uint8_t* qt = xmalloc(C * Rp); uint8_t* st = xmalloc(C * Rp / 32);
  CHECK(oracle_mxfp8_quant_row(x, R, C, C, q, s) == 0);
  CHECK(oracle_mxfp8_quant_colT(x, R, C, C, qt, st) == 0);
  double* d = xmalloc(sizeof(double) * R * Cp);
  oracle_mxfp8_dequant(q, s, R, Cp, d);
  double* Cm = xmalloc(sizeof(double) * R * R); double* Ca = xmalloc(sizeof(double) * R * R);
  CHECK(oracle_gemm(q, s, q, s, R, R, Cp, Cm, Ca) == 0);
  int64_t mi[3] = {0, R - 1, R / 2}, ni[3] = {R - 1, 0, R / 3};
  double cs[3], cas[3];
  CHECK(oracle_gemm_sampled(q, s, q, s, R, R, Cp, mi, ni, 3, cs, cas) == 0);
  /* grouped token-axis copy over groups with empty, single and ragged sizes */
  int32_t ge[5];
  int32_t sizes[5] = {0, 1, (int32_t)(R / 3), 0, 0};
  sizes[4] = (int32_t)(R - sizes[1] - sizes[2]);
  int64_t acc = 0, need = 0;
  for (int g = 0; g < 5; g++) { acc += sizes[g]; ge[g] = (int32_t)acc; need += (sizes[g] + 31) / 32 * 32; }
  int64_t ldq = (need + 31) / 32 * 32 + 32;
  uint8_t* qg = xmalloc(C * ldq); uint8_t* sg = xmalloc(C * ldq / 32);
  CHECK(oracle_mxfp8_quant_grouped_colT(x, R, C, C, ge, 5, ldq, qg, sg) == 0);
  double* Ck = xmalloc(sizeof(double) * 5 * C * C); double* Cka = xmalloc(sizeof(double) * 5 * C * C);
  CHECK(oracle_grouped_gemm_ragged_k(qg, sg, qg, sg, C, C, ldq, ge, 5, Ck, Cka) == 0);
  /* ragged M: rows of X by group, B = 5 experts of C rows */
  uint8_t* Bq = xmalloc(5 * C * Cp); uint8_t* Bs = xmalloc(5 * C * Cp / 32);
  for (int g = 0; g < 5; g++) {
    uint16_t* w = xmalloc(sizeof(uint16_t) * C * C);
    for (int64_t i = 0; i < C * C; i++) w[i] = rand_bf16();
    CHECK(oracle_mxfp8_quant_row(w, C, C, C, Bq + g * C * Cp, Bs + g * C * Cp / 32) == 0);
    free(w);
  }
  double* Cr = xmalloc(sizeof(double) * R * C); double* Cra = xmalloc(sizeof(double) * R * C);
  CHECK(oracle_grouped_gemm_ragged_m(q, s, Bq, Bs, R, C, Cp, ge, 5, Cr, Cra) == 0);
  /* malformed group ends are rejected, never read past */
  int32_t bad[3] = {(int32_t)R, 0, (int32_t)R + 5};
  CHECK(oracle_mxfp8_quant_grouped_colT(x, R, C, C, bad, 3, ldq, qg, sg) != 0);
  CHECK(oracle_grouped_gemm_ragged_m(q, s, Bq, Bs, R, C, Cp, bad, 3, Cr, Cra) != 0);
  CHECK(oracle_grouped_gemm_ragged_k(qg, sg, qg, sg, C, C, ldq, bad, 3, Ck, Cka) != 0);
  CHECK(oracle_mxfp8_quant_row(x, R, C, C - 1, q, s) != 0);
  free(x); free(q); free(s); free(qt); free(st); free(d); free(Cm); free(Ca); free(qg); free(sg);
  free(Ck); free(Cka); free(Bq); free(Bs); free(Cr); free(Cra);
  return 0;
}

static int fp4(int64_t rows, int64_t L, float sf) {
  int64_t Lp = (L + 31) / 32 * 32;
  float* x = xmalloc(sizeof(float) * rows * L);
  float* y = xmalloc(sizeof(float) * rows * L);
  for (int64_t i = 0; i < rows * L; i++) x[i] = ldexpf((float)((int32_t)next() % 1000) / 97.0f, (int)(next() % 40) - 20);
  uint8_t* codes = xmalloc(rows * Lp / 2); uint8_t* sc = xmalloc(rows * Lp / 32); uint8_t* mask = xmalloc(rows * Lp / 8);
  CHECK(oracle_mxfp4_qdq_ex(x, y, rows, L, sf, codes, sc, mask) == 0);
  float* gx = xmalloc(sizeof(float) * rows * L);
  oracle_mxfp4_ste_backward(y, mask, gx, rows, L);
  double* d = xmalloc(sizeof(double) * rows * Lp);
  oracle_mxfp4_dequant(codes, sc, rows, Lp, d);
  double* C = xmalloc(sizeof(double) * rows * rows); double* Ca = xmalloc(sizeof(double) * rows * rows);
  CHECK(oracle_gemm_fp4(codes, sc, codes, sc, rows, rows, Lp, C, Ca) == 0);
  CHECK(oracle_mxfp4_qdq_ex(x, y, rows, L, -1.0f, NULL, NULL, NULL) != 0);
  free(x); free(y); free(codes); free(sc); free(mask); free(gx); free(d); free(C); free(Ca);
  return 0;
}

int main(void) {
  const int64_t S[][2] = {{1, 1}, {1, 32}, {2, 33}, {33, 2}, {3, 17}, {65, 65}, {70, 130}};
  for (size_t i = 0; i < sizeof S / sizeof S[0]; i++)
    if (shapes(S[i][0], S[i][1])) return 1;
  if (fp4(2, 33, 6.0f) || fp4(3, 17, 5.0f) || fp4(48, 33, 7.25f) || fp4(1, 1, 6.0f)) return 1;
  printf("ok\n");
  return 0;
}
