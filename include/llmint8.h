/*
 * llmint8 -- the LLM.int8() matrix multiply on AMD Instinct MI355X (gfx950).
 *
 * The operation ("LLM.int8(): 8-bit Matrix Multiplication for Transformers at Scale",
 * abstract): a two-part procedure for the feed-forward and attention projection
 * products Y = X W.
 *   1. Vector-wise quantization: one normalization constant per inner-product vector,
 *      i.e. per row of X (token) and per output column of W.  The constant is the
 *      vector's absolute maximum s (kept in fp32); a value x is coded as
 *      q = clamp(round_half_even(x * RN32(127/s)), -127, 127)  (s = 0 gives q = 0).
 *   2. Mixed-precision decomposition: the feature dimensions of X that hold outliers
 *      -- every column j with |X[i,j]| > threshold for some row i of this call
 *      (talk summary "llama3-model-quantization", "Understanding Outliers in
 *      Transformer Models": outliers sit in specific columns of the input batch) --
 *      go through a 16-bit matrix multiplication; everything else goes through int8
 *      with exact int32 accumulation.
 *   With O the ascending outlier set, Xq the int8 codes of X with the columns in O
 *   zeroed (row scales s_x taken over the other columns), Wq the int8 codes of W
 *   (column scales s_w), C = Xq Wq^T (int32) and F = X[:,O] Wq[:,O]^T (16-bit inputs,
 *   fp32 accumulation; Wq's codes are exact in fp16/bf16), each element of Y is
 *       y = RN32( RN32( RN32((float)C * r_i) * c_n ) + RN32(c_n * F) ),
 *       r_i = RN32(s_x[i] / 127),  c_n = RN32(s_w[n] / 127),  Y = round_even_to_T(y),
 *   i.e. the int32 product dequantized by the outer product of the two scale vectors
 *   divided by 127^2, plus the outlier product.  (Rounding to nearest: "nuQmm" report
 *   page, GPTQ statement under "Large-model Quantization".)
 *
 * Conventions for every call below.
 *   - Pointers are DEVICE pointers owned by the caller unless marked HOST.  The library
 *     allocates no memory and keeps no state between calls; it is re-entrant.  (The one
 *     exception, int8_matmul_noalloc at the end, works in a static device array of the
 *     library's own instead of a caller workspace.)
 *   - `stream` is a hipStream_t (NULL: the default stream).  Calls only enqueue work on
 *     it and return before it runs, except int8_matmul_stats, which synchronizes it.
 *   - `dtype` is LLMINT8_F16 or LLMINT8_BF16; X, W and Y share it.
 *   - Returns LLMINT8_OK (0) or a negative status.  Every argument is validated before
 *     any GPU work is enqueued; on a validation error nothing is written.  A HIP error
 *     is returned as LLMINT8_EHIP (the sticky error is consumed); work enqueued before
 *     it may have run.  No C++ exception crosses this interface.
 *   - Shapes: M >= 0 rows of X (tokens), K >= 0 features, N >= 0 output columns;
 *     K must be a multiple of 16 and N a multiple of 8; K <= 133143 so that every
 *     int32 dot product is exact (127 * 127 * K < 2^31), else LLMINT8_ERANGE.
 *     Any M (ragged tails included); M, N, K < 2^31.
 *   - Layouts are row-major.  X: M x K.  W: K x N.  Wq: N x K (K contiguous).  Y: M x N.
 *     X, W, Wq, Y and the workspace must be 16-byte aligned; w_scale 4-byte aligned.
 *   - Non-finite inputs, and nonzero vectors whose absmax is below 2^-120 (where
 *     127/s overflows fp32; bf16 only), are outside the contract.
 *   - Environment (read on every call, host side only):
 *       LLMINT8_LOG=1        prints each call's sizes, dtype, threshold, path (tiled or
 *                            small batch) and each launch ("stage") to stderr.
 *       LLMINT8_FAULT=<stage> test switch, a dry run: nothing is enqueued; each stage the
 *                            call reaches before the named one is taken as done and the
 *                            named one as failed, so the call returns LLMINT8_EHIP and
 *                            reports nothing as done (int8_matmul_stats leaves its host
 *                            output unwritten).  A call whose path lacks that stage returns
 *                            LLMINT8_OK without having enqueued anything.  Stage names are
 *                            the ones LLMINT8_LOG prints (detect, compact, code_rows,
 *                            xpass_small, gemm, gemm_small, weight, list_bitmap, gather_wo,
 *                            stats_copy, stats_sync, stats_copy_cols, group_colmax,
 *                            quantize_weight_groups, group_xpass, gemm_group,
 *                            gemm_group_small, fill_zero, block_quantize, block_dequantize,
 *                            scratch_symbol).
 */
#ifndef LLMINT8_H
#define LLMINT8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum llmint8_dtype { LLMINT8_F16 = 0, LLMINT8_BF16 = 1 };

enum llmint8_status {
    LLMINT8_OK = 0,
    LLMINT8_EINVAL = -1,     /* bad pointer, shape, alignment, dtype, threshold or aliasing */
    LLMINT8_EWORKSPACE = -2, /* workspace missing, misaligned or smaller than required     */
    LLMINT8_EHIP = -3,       /* a HIP launch or runtime call failed                        */
    LLMINT8_ERANGE = -4      /* K too large for exact int32 accumulation                   */
};

/* Human-readable name of a status code (static string, never NULL). */
const char* llmint8_status_string(int status);

/*
 * Offline weight conversion ("LLM.int8()" page, abstract: a 16-bit checkpoint is
 * loaded, converted to Int8 and used immediately; data-free, one pass -- "nuQmm"
 * report page, GPTQ statement under "The Gptq Algorithm", on round-to-nearest).
 *   W        in : K x N, dtype, row-major.
 *   Wq       out: N x K int8, row-major (each output column's codes contiguous).
 *   w_scale  out: fp32[N], s_w[n] = max_k |W[k,n]|.
 * K = 0 gives w_scale = 0; N = 0 is a no-op.
 */
int int8_quantize_weight(const void* W, int64_t K, int64_t N, int dtype,
                         int8_t* Wq, float* w_scale, void* stream);

/* Bytes of device workspace int8_matmul needs for these sizes (worst case: every
 * column an outlier).  int8_matmul_stats needs int8_matmul_workspace_bytes(M, K, 0). */
size_t int8_matmul_workspace_bytes(int64_t M, int64_t K, int64_t N);

/*
 * The LLM.int8() product Y = X W (see the top of this file for the exact definition).
 *   X          in : M x K, dtype.
 *   Wq, w_scale in: from int8_quantize_weight (N x K int8, fp32[N]).
 *   threshold  in : outlier threshold tau >= 0 (+INFINITY allowed: no outliers;
 *                   0: every nonzero column is an outlier, the 16-bit product).
 *                   NaN or negative: LLMINT8_EINVAL.
 *   Y          out: M x N, dtype.  Must not overlap X, Wq, w_scale or the workspace.
 *   workspace  scratch of at least int8_matmul_workspace_bytes(M, K, N) bytes,
 *              16-byte aligned.  After the call it holds the X pass's products in the
 *              layout int8_matmul_workspace_layout describes (Xq, s_x, O, n_O, X[:,O]).
 */
int int8_matmul(const void* X, int64_t M, int64_t K, int dtype,
                const int8_t* Wq, const float* w_scale, int64_t N,
                float threshold, void* Y,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * The outlier feature dimensions of X for this threshold ("LLM.int8()" page,
 * abstract: more than 99.9% of values are multiplied in 8-bit; this reports the rest).
 *   n_outlier_cols  HOST out: n_O = |O|.
 *   outlier_cols    DEVICE out, may be NULL, capacity K int32: O in ascending order.
 * Synchronizes `stream`.  Workspace: int8_matmul_workspace_bytes(M, K, 0) bytes.
 */
int int8_matmul_stats(const void* X, int64_t M, int64_t K, int dtype, float threshold,
                      int32_t* n_outlier_cols, int32_t* outlier_cols,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * The two stages int8_matmul runs, for callers that reuse one X pass.
 *   int8_matmul_prepare:  the X pass -- outlier set O and n_O, row scales s_x, int8
 *                         codes Xq with the outlier columns zeroed, and the compact
 *                         16-bit outlier operands X[:,O] and Wq[:,O] -- into the
 *                         workspace (layout: int8_matmul_workspace_layout).  Wq may be
 *                         NULL when N == 0.
 *   int8_matmul_products: C = Xq Wq^T (int8, int32 accumulation), F = X[:,O] Wq[:,O]^T
 *                         (16-bit, fp32 accumulation) and the dequantizing epilogue,
 *                         from a workspace prepared for the same X, Wq, M, K, N, dtype
 *                         and threshold on the same stream.  It may be called again on
 *                         the same prepared workspace; the calls then follow each other on
 *                         one stream (with few output tiles the products split their K
 *                         stages over the GPU and exchange exact int32 partial sums through
 *                         the workspace's scratch, so concurrent calls on one workspace race).
 * int8_matmul(X, ...) == int8_matmul_prepare(X, ...) then int8_matmul_products(...).
 * Same conventions and status codes as int8_matmul.
 */
int int8_matmul_prepare(const void* X, int64_t M, int64_t K, int dtype, const int8_t* Wq, int64_t N,
                        float threshold, void* workspace, size_t workspace_bytes, void* stream);

int int8_matmul_products(int64_t M, int64_t K, int dtype, const int8_t* Wq, const float* w_scale, int64_t N,
                         void* Y, void* workspace, size_t workspace_bytes, void* stream);

/* Where int8_matmul leaves the X pass's products in its workspace (byte offsets from
 * the workspace start; pitches in elements).  All regions are 256-byte aligned.
 *   xq        int8  [M][xq_pitch]   Xq; columns in O are 0; columns >= K are 0
 *   s_x       fp32  [M]             row absmax over the non-outlier columns
 *   n_outliers int32                n_O
 *   outliers  int32 [K]             O ascending (first n_O entries valid)
 *   xo        dtype [M][xo_pitch]   X[:, O] (first n_O columns; zero up to the next
 *                                   multiple of 32)
 *   wo        dtype [N][xo_pitch]   Wq[:, O] cast to dtype (same padding); written only by
 *                                   the tiled path -- the small-batch product kernel
 *                                   gathers these values itself
 *   scratch   internal (outlier flags; up to 112 rows, and for small batches, per-row
 *             partial maxima; for small batches from 8 rows up, a copy of Xq in the
 *             product kernel's operand blocks)
 *   total     bytes (int8_matmul_workspace_bytes)
 *   small_batch  1 when these sizes take the small-batch path (M <= 128, K <= 65536 and
 *             N small enough that streaming Wq once beats the tiled kernel), else 0 */
typedef struct {
    size_t xq, xq_pitch, s_x, n_outliers, outliers, xo, xo_pitch, wo, scratch, total, small_batch;
} llmint8_workspace_layout;

int int8_matmul_workspace_layout(int64_t M, int64_t K, int64_t N, llmint8_workspace_layout* out);

/*
 * Test hook, not part of the product path: the same kernels as int8_matmul with the
 * epilogue replaced by a store of the raw accumulators, so that the int32 product can
 * be compared exactly.
 *   C  out: M x N int32, C = Xq Wq^T.
 *   F  out: M x N fp32, the 16-bit outlier product (0 where there are no outliers).
 */
int int8_matmul_accumulators(const void* X, int64_t M, int64_t K, int dtype,
                             const int8_t* Wq, int64_t N, float threshold,
                             int32_t* C, float* F,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Fixed (caller-supplied) outlier dimensions.  The outlier feature dimensions are
 * systematic and context-independent (talk summary "llama3-model-quantization",
 * "Understanding Outliers in Transformer Models"), so a caller may fix the set O offline
 * (for example from calibration) instead of detecting it per call; their rows of W are
 * then kept in 16 bits (the HN discussion on the "LLM.int8()" page: outliers kept in
 * their original precision).  O: n_O column indices of X (= row indices of W), strictly
 * ascending, in [0, K) -- otherwise the result is undefined (entries outside [0, K) are
 * ignored; no access leaves the buffers).  W_O: N x P 16-bit, P = n_O rounded up to a
 * multiple of 32, row-major, zero past n_O.
 *
 * Weight conversion: s_w[n] = max over k not in O of |W[k,n]|; Wq[n,k] = 0 for k in O,
 * else the code of the conversion above; W_O[n,t] = W[O[t], n] exactly.
 *   outlier_cols  device int32[n_O], 4-byte aligned; n_outlier_cols in [0, K].
 *   workspace     >= int8_quantize_weight_fixed_workspace_bytes(K) bytes, 16-byte aligned.
 */
size_t int8_quantize_weight_fixed_workspace_bytes(int64_t K);
int int8_quantize_weight_fixed(const void* W, int64_t K, int64_t N, int dtype, const int32_t* outlier_cols,
                               int64_t n_outlier_cols, int8_t* Wq, float* w_scale, void* W_O, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * The product with the fixed set: no detection; the X pass codes every row against O (s_x
 * over the columns not in O, Xq zero on O, X[:,O] gathered), then
 *   y = RN32( RN32( RN32((float)C * r_i) * c_n ) + F ),   F = X[:,O] W_O^T
 * (16-bit inputs, fp32 accumulation; the exact W rows, so the term is not scaled by c_n).
 * Arguments as int8_matmul, plus outlier_cols / n_outlier_cols / W_O as above; the
 * workspace is int8_matmul_workspace_bytes(M, K, N) and afterwards holds the X pass's
 * products (its W_O region is unused).  No threshold is involved.
 */
int int8_matmul_fixed(const void* X, int64_t M, int64_t K, int dtype, const int32_t* outlier_cols,
                      int64_t n_outlier_cols, const int8_t* Wq, const float* w_scale, const void* W_O, int64_t N,
                      void* Y, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Block-wise absmax int8 codec of a flat fp32 tensor ("llama3-model-quantization" talk
 * summary, Key Points, 8-bit optimizers: the optimizer state is cut into blocks, each
 * block is normalised by its own maximum and kept as 8-bit values; the linear code is
 * read, with the quantizer of the matmul above).  Block b holds elements
 * [b*block, min((b+1)*block, n)) (the last block may be short):
 *   absmax[b] = max |x| over the block (fp32),
 *   q[i] = clamp(round_half_even(RN32(x[i] * RN32(127 / absmax[b]))), -127, 127)
 *          (absmax 0: q = 0),
 *   decode x'[i] = RN32((float)q[i] * RN32(absmax[b] / 127)).
 *   x       : n fp32 values (device), 16-byte aligned.
 *   q       : n int8 codes (device), 4-byte aligned.
 *   absmax  : ceil(n / block) fp32 (device), 4-byte aligned.
 *   block   : a power of two in [64, 4096], else LLMINT8_EINVAL.
 * n = 0 is a no-op.  Inputs and outputs must not overlap (LLMINT8_EINVAL).  Non-finite
 * values are outside the contract.
 */
int int8_blockwise_quantize(const float* x, int64_t n, int64_t block, int8_t* q, float* absmax, void* stream);
int int8_blockwise_dequantize(const int8_t* q, const float* absmax, int64_t n, int64_t block, float* x,
                              void* stream);

/*
 * Group-wise scales along K: the finer granularity than one scale per row or column that
 * the "nuQmm" report page names (its citation snippets on nuQmm/ZeroQuant and on GPTQ's
 * grouping, with groups of 1024 weights), applied here to both operands and without the
 * outlier decomposition.  K is cut into ng = K / G groups of G consecutive features:
 *   s_x[i*ng + g] = max |X[i,k]| over group g of row i, Xq = the code of that group,
 *   s_w[n*ng + g] = max |W[k,n]| over group g of column n, Wq = the code of that group
 *   (the quantizer of the vector-wise conversion: clamp(rne(RN32(x * RN32(127/s))), ±127),
 *   s = 0 codes 0), and
 *   y[i,n] = sum over g ascending, in fp32:
 *            acc = RN32(acc + RN32(RN32((float)C_g * RN32(s_x/127)) * RN32(s_w/127))),
 *   C_g = the exact int32 product of the group's codes;  Y = RN_T(acc).
 *   group : G, a power of two in [128, 4096] that divides K, else LLMINT8_EINVAL
 *           (any value is accepted when K = 0).
 *
 * Weight conversion: Wq N x K int8 (16-byte aligned), w_scale N x ng fp32 row-major.
 * Shape rules, dtype and alignments as int8_quantize_weight.
 */
int int8_quantize_weight_group(const void* W, int64_t K, int64_t N, int dtype, int64_t group, int8_t* Wq,
                               float* w_scale, void* stream);

/*
 * The group-wise product.  Workspace: int8_matmul_group_workspace_bytes(M, K, group)
 * bytes, 256-byte aligned (0 if the arguments are invalid).  After a call with M, N and
 * K nonzero it holds the X pass's products: Xq (M x K int8, row-major) at offset 0, s_x
 * (M x ng fp32, row-major) at offset round_up(M*K, 256), and the dequantization factors
 * RN32(s_x/127) transposed (ng x M) after that.  Y: M x N of X's dtype, 16-byte aligned.
 * M = 0 or N = 0 is a no-op; K = 0 gives Y = 0 (the workspace is then not needed).
 * Inputs, Y and the workspace must not overlap (LLMINT8_EINVAL).
 */
size_t int8_matmul_group_workspace_bytes(int64_t M, int64_t K, int64_t group);
/* Which product kernel int8_matmul_group runs for these sizes: 1 the small-batch (split-N,
 * weight-streaming) kernel, 0 the tiled one; a negative status for invalid sizes. */
int int8_matmul_group_small_batch(int64_t M, int64_t K, int64_t N, int64_t group);
int int8_matmul_group(const void* X, int64_t M, int64_t K, int dtype, int64_t group, const int8_t* Wq,
                      const float* w_scale, int64_t N, void* Y, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * int8_matmul_group in two calls on one workspace, as int8_matmul_prepare / _products: the
 * X pass (codes, scales and factors of X's row groups) and then the products with their
 * per-group dequantization.  The products read only the workspace, Wq and w_scale, so one
 * X pass can serve several weights of the same K and group size.
 */
int int8_matmul_group_prepare(const void* X, int64_t M, int64_t K, int dtype, int64_t group, void* workspace,
                              size_t workspace_bytes, void* stream);
int int8_matmul_group_products(int64_t M, int64_t K, int dtype, int64_t group, const int8_t* Wq,
                               const float* w_scale, int64_t N, void* Y, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * int8_matmul without a caller workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Arguments, result and status codes are int8_matmul's, minus the workspace: the same
 * kernels run on a scratch array the library keeps in device memory,
 * LLMINT8_NOALLOC_SCRATCH_BYTES bytes on every GPU the library runs on, held until the
 * process ends.  The call allocates nothing (no hipMalloc, no allocating library routine);
 * its first call on a device looks up that device's copy of the array.
 *   Sizes: int8_matmul_workspace_bytes(M, K, N) must not exceed
 *          LLMINT8_NOALLOC_SCRATCH_BYTES, else LLMINT8_EWORKSPACE and nothing is enqueued.
 *          Small batches (M <= 128 on the small-batch path: e.g. 16 x 8192 x 8192 needs
 *          under 1 MiB) fit; so do tiled calls of moderate size (the tiled path reserves
 *          the worst case of every column an outlier, 2 N K bytes for the gathered weight
 *          columns alone, and with few output tiles 512 KB of int32 partial sums per
 *          workgroup of its K split).
 *   Concurrency: every call on one GPU works in that GPU's single array.  Calls that
 *          overlap in time on one GPU (on different streams or host threads) race and
 *          give undefined results; calls ordered on one stream are safe.  The array keeps
 *          the last call's contents; no call needs any of it to start at zero.
 */
#define LLMINT8_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int int8_matmul_noalloc(const void* X, int64_t M, int64_t K, int dtype, const int8_t* Wq, const float* w_scale,
                        int64_t N, float threshold, void* Y, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* LLMINT8_H */
