/*
 * CPU oracle for the LLM.int8() matrix multiply -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the CPU-baseline leg of the benchmark
 * may call, link or load this code.  The GPU library never does, and this code
 * shares nothing with it (no headers, no helpers, no tables).
 *
 * What it computes (plain, slow, in the order the method states it):
 *   "LLM.int8(): 8-bit Matrix Multiplication for Transformers at Scale", abstract:
 *     (1) vector-wise quantization -- one normalization constant per inner-product
 *         vector: per row of X (token) and per output column of W;
 *     (2) mixed-precision decomposition -- the outlier feature dimensions of X go
 *         through a 16-bit matrix multiplication, everything else through int8.
 *   Readings where the pages are silent (each is listed in the design notes):
 *     - scale = absmax of the vector, stored as fp32; the absmax maps to +-127
 *       (talk summary "llama3-model-quantization", Key Points: normalise by the
 *       block's maximum value);
 *     - rounding = round to nearest, ties to even ("nuQmm" report page, GPTQ
 *       statement under "Large-model Quantization": RTN);
 *     - outlier dimension j  <=>  some row i has |X[i,j]| > tau (strict), over the
 *       whole batch (talk summary, "Understanding Outliers in Transformer Models":
 *       outliers sit in specific columns of the input batch);
 *     - the row scale of X is taken over the non-outlier columns only;
 *     - the 16-bit W rows of the outlier part are the int8 codes cast exactly to
 *       the 16-bit type, with the column scale applied in the epilogue;
 *     - epilogue, every op rounded to fp32 once, no fused multiply-add:
 *         r_i = s_x[i]/127, c_n = s_w[n]/127,
 *         y = ((float)C*r_i)*c_n + c_n*F,   Y = round_to_T(y).
 *
 * Parity pins: every function here is checked by tests that do not re-type it
 * (brute force, closed forms on exactly representable lattices, exhaustive
 * quantizer sweeps, symmetry invariants, library conversions).
 */
#ifndef LLMINT8_ORACLE_H
#define LLMINT8_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_F16 = 0, ORC_BF16 = 1 };

/* Thread count used by the row-parallel loops (<= 0: all host cores). Returns the count in effect. */
int orc_set_threads(int n);

/* 16-bit <-> fp32 conversions (widening is exact; narrowing rounds to nearest-even,
 * fp16 overflow -> +-inf).  Bulk forms for the tests. */
float orc_to_f32(uint16_t h, int dt);
uint16_t orc_from_f32(float f, int dt);
void orc_to_f32_n(const uint16_t* h, int64_t n, int dt, float* out);
void orc_from_f32_n(const float* f, int64_t n, int dt, uint16_t* out);

/* The scalar quantizer: inv = s > 0 ? RN32(127/s) : 0 ;  q = clamp(rne(RN32(x*inv)), -127, 127). */
float orc_inv_scale(float s);
int8_t orc_quantize(float x, float inv);
void orc_quantize_n(const float* x, int64_t n, float s, int8_t* q);

/* Offline weight conversion.  W: K x N row-major (16-bit, dtype dt).
 * Out: Wq N x K row-major (K contiguous), s_w[N] = column absmax. */
void orc_quantize_weight(const uint16_t* W, int64_t K, int64_t N, int dt, int8_t* Wq, float* s_w);

/* Outlier feature dimensions: ascending list O of every column j with |X[i,j]| > tau
 * for some row i.  X: M x K row-major.  Returns n_O; O needs capacity K. */
int64_t orc_outlier_columns(const uint16_t* X, int64_t M, int64_t K, int dt, float tau, int32_t* O);

/* Row quantization with the outlier columns removed, and the outlier gather.
 * Out: Xq M x K (0 in outlier columns), s_x[M], XO M x nO (exact copies, 16-bit bits). */
void orc_quantize_rows(const uint16_t* X, int64_t M, int64_t K, int dt, const int32_t* O, int64_t nO,
                       int8_t* Xq, float* s_x, uint16_t* XO);

/* Int8 part, exact: C[r,n] = sum_k Xq[rows[r],k] * Wq[n,k] for the listed rows
 * (rows == NULL: rows 0..nrows-1).  Returns 0, or -1 if a sum leaves int32. */
int orc_int_gemm(const int8_t* Xq, const int8_t* Wq, int64_t K, int64_t N,
                 const int64_t* rows, int64_t nrows, int32_t* C);

/* 16-bit outlier part: F[r,n] = fp32 sum over t ascending of XO[i,t] * (T)Wq[n,O[t]],
 * i = rows[r].  Also the float64 sum F64 and the absolute sum A (both may be NULL). */
void orc_outlier_gemm(const uint16_t* XO, int64_t nO, int dt, const int8_t* Wq, int64_t K, int64_t N,
                      const int32_t* O, const int64_t* rows, int64_t nrows,
                      float* F, double* F64, double* A);

/* Dequantizing epilogue for nrows rows: s_x_rows[r] is the row scale of row r.
 * Out: y (fp32, may be NULL) and Y (16-bit bits). */
void orc_dequant(const int32_t* C, const float* F, const float* s_x_rows, const float* s_w,
                 int64_t nrows, int64_t N, int dt, float* y, uint16_t* Y);

/* Fixed outlier dimensions (caller-supplied, e.g. found offline: the talk summary,
 * "Understanding Outliers in Transformer Models", calls the outlier dimensions systematic
 * and context-independent; the HN discussion on the "LLM.int8()" page describes the
 * outliers as kept in their original precision).  O: n_O distinct column indices of X /
 * row indices of W, ascending.
 * Weight conversion with O fixed: s_w[n] = max over k not in O of |W[k,n]|; Wq[n,k] = 0
 * for k in O, else the code above; WO[n * nO + t] = W[O[t], n] (exact 16-bit copy). */
void orc_quantize_weight_fixed(const uint16_t* W, int64_t K, int64_t N, int dt, const int32_t* O, int64_t nO,
                               int8_t* Wq, float* s_w, uint16_t* WO);

/* Outlier product with the exact 16-bit rows: F[r,n] = sum over t ascending of
 * (float)XO[row r, t] * (float)WO[n, t] in fp32 (each product exact), F64 in double, A the
 * sum of |products|. */
void orc_outlier_gemm_exact(const uint16_t* XO, int64_t nO, int dt, const uint16_t* WO, int64_t N,
                            const int64_t* rows, int64_t nrows, float* F, double* F64, double* A);

/* Epilogue with the unscaled outlier part: y = RN32(RN32(RN32((float)C * r_i) * c_n) + F). */
void orc_dequant_fixed(const int32_t* C, const float* F, const float* s_x_rows, const float* s_w,
                       int64_t nrows, int64_t N, int dt, float* y, uint16_t* Y);

/* Group-wise scales along K (the finer granularity the "nuQmm" report page discusses for
 * weight quantization: one scale per group of consecutive input features; here for both
 * operands, no outlier decomposition).  G divides K; ng = K / G groups.
 *   s_x[i*ng + g] = max |X[i,k]| over k in [gG, (g+1)G);  Xq[i,k] = code with that scale;
 *   s_w[n*ng + g] = max |W[k,n]| over the same k;          Wq[n,k] = code with that scale;
 *   C_g[i,n] = sum over the group of Xq Wq (exact int32);
 *   acc = 0; for g ascending: acc = RN32(acc + RN32(RN32((float)C_g * r_ig) * c_ng)),
 *   r_ig = RN32(s_x/127), c_ng = RN32(s_w/127);  Y = RN_T(acc). */
void orc_group_quantize_rows(const uint16_t* X, int64_t M, int64_t K, int dt, int64_t G, int8_t* Xq, float* s_x);
void orc_group_quantize_weight(const uint16_t* W, int64_t K, int64_t N, int dt, int64_t G, int8_t* Wq, float* s_w);
void orc_group_gemm(const int8_t* Xq, const float* s_x, const int8_t* Wq, const float* s_w, int64_t K, int64_t N,
                    int64_t G, const int64_t* rows, int64_t nrows, int dt, float* y, uint16_t* Y);

/* Block-wise absmax int8 codec of a flat fp32 tensor ("llama3-model-quantization" talk
 * summary, Key Points, 8-bit optimizers: the state is cut into blocks, each block is
 * normalised by its own maximum and stored as 8-bit values; the linear code is read, the
 * same quantizer as above).  Block b = elements [b*block, min((b+1)*block, n)):
 *   absmax[b] = max |x| over the block,
 *   q = clamp(rne(RN32(x * RN32(127 / absmax[b]))), -127, 127)   (absmax 0: q = 0),
 *   decode: x' = RN32((float)q * RN32(absmax[b] / 127)). */
void orc_block_quantize(const float* x, int64_t n, int64_t block, int8_t* q, float* absmax);
void orc_block_dequantize(const int8_t* q, const float* absmax, int64_t n, int64_t block, float* x);

#ifdef __cplusplus
}
#endif
#endif
