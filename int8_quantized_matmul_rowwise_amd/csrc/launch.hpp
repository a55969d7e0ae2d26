// Internal launchers of the llmint8 kernels (host side).  Each enqueues on `stream`
// and returns the launch status; shapes were validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace llmint8 {

// ---- weight conversion
// Column absmax partials over `splits` slices of K, then the final scale + the
// quantize-transpose into Wq (N x K).
int64_t weight_splits(int64_t K);
hipError_t launch_weight(int dt, const void* W, int64_t K, int64_t N, int8_t* Wq, float* w_scale,
                         const uint32_t* skip /* nullable: rows of W (outlier set) to leave out */,
                         hipStream_t stream);
// p[0, n) = 0 (a kernel, not a memset node, so that the call can be captured in a graph)
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t stream);
// W_O (N x P, 16-bit): W[O[t], n] for t < nO, zero up to P.
hipError_t launch_gather_wo(const void* W, int64_t K, int64_t N, const int32_t* O, int64_t nO, int64_t P, void* WO,
                            hipStream_t stream);
// The bitmap of a caller's column list (single workgroup), as one row-block partial for
// launch_compact: the fixed-outlier paths then share the compaction and the row coding.
hipError_t launch_list_bitmap(int64_t K, const int32_t* O, int64_t nO, uint32_t* partial, hipStream_t stream);

// ---- X pass
int64_t detect_row_blocks(int64_t M);
hipError_t launch_detect(int dt, const void* X, int64_t M, int64_t K, float tau, uint32_t* partial,
                         hipStream_t stream);
hipError_t launch_compact(int64_t M, int64_t K, const uint32_t* partial, uint32_t* bitmap, int32_t* O,
                          int32_t* n_out, hipStream_t stream);

// Small-batch path (slab X pass, split-N product kernel), for M <= kSmallM and K <= kSmallK
// where it beats the tiled path.  The split-N kernel streams Wq once at about 5 TB/s, and
// every row of X adds to that time (its re-reads of Xq from the cache): about 2.2 % per
// row up to 64 rows (two column groups per workgroup), about 5 % beyond (one); the tiled
// kernel, with one 256-row tile, takes about K * 10.5 ns per round of 256-column tiles
// over the compute units, whatever M.  Measured on MI355X (256 CUs), M = 16 to 128 on
// N x K = 36864 x 12288, 28672 x 8192, 16384 x 53248, 16384 x 4096, 14336 x 4096,
// 8192 x 8192 and 4096 x 4096: N * (1 + c M) / 5 TB/s < K * 10.5 ns * rounds, the test
// below, picks the faster path in each of those cases, or one within 2 %.
constexpr int64_t kSmallM = 128;
constexpr int64_t kSmallK = 65536;
constexpr int64_t kRoutingCUs = 256;
inline bool small_batch(int64_t M, int64_t K, int64_t N) {
    if (M > kSmallM || K > kSmallK) return false;
    const int64_t rounds = ((N + 255) / 256 + kRoutingCUs - 1) / kRoutingCUs;
    const int64_t c = M <= 64 ? 22 : 50;  // per mille of the Wq stream time per row
    return N * (1000 + c * M) < 52500000 * (rounds > 0 ? rounds : 1);
}

struct XPassArgs {
    int dt;
    const void* X;
    float tau;
    int64_t M, K, N;
    const uint32_t* bitmap;
    const int32_t* O;
    const int32_t* n_out;
    int8_t* Xq;
    int64_t xq_pitch;
    float* s_x;
    void* XO;
    int64_t xo_pitch;
    const int8_t* Wq;  // NULL: no W_O gather
    void* WO;
};
hipError_t launch_code_rows(const XPassArgs& a, const uint32_t* bitmap, int32_t* O, int32_t* n_out,
                            hipStream_t stream);
// pmax (M x ceil(K/512) words of scratch): per row and 512-column slab, the slab's
// maximum over its non-outlier columns
hipError_t launch_xpass_small(const XPassArgs& a, int32_t* O, int32_t* n_out, uint32_t* bitmap, uint32_t* pmax,
                              hipStream_t stream);

// ---- products + epilogue
struct GemmArgs {
    int dt;
    const int8_t* Xq;
    int64_t xq_pitch;
    const int8_t* Wq;
    int64_t M, N, K;
    const float* s_x;
    const float* s_w;
    const void* XO;
    const void* WO;     // 16-bit outlier rows of W, N x wo_pitch (the small-batch kernel
                        // gathers them from Wq itself when f_scaled)
    int64_t xo_pitch;
    int64_t wo_pitch;
    bool f_scaled;      // W_O holds Wq's codes (the outlier term is scaled by c_n) or exact
                        // 16-bit W rows (fixed outlier set: unscaled)
    const int32_t* n_out;
    const int32_t* O;   // outlier columns
    void* Y;          // product path
    int32_t* C_acc;   // accumulator dump (test hook); Y == NULL then
    float* F_acc;
};
hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream);
hipError_t launch_gemm_small(const GemmArgs& a, hipStream_t stream);

// ---- block-wise absmax int8 codec of a flat fp32 tensor
bool codec_block_ok(int64_t block);  // a power of two in [64, 4096]
hipError_t launch_block_quantize(const float* x, int64_t n, int64_t block, int8_t* q, float* absmax,
                                 hipStream_t stream);
hipError_t launch_block_dequantize(const int8_t* q, const float* absmax, int64_t n, int64_t block, float* x,
                                   hipStream_t stream);

// ---- group-wise scales along K (G a power of two in [128, 4096] dividing K)
bool group_size_ok(int64_t G, int64_t K);
// s_w[n*ng + g] = absmax of column n of W over rows [g*G, (g+1)*G)
hipError_t launch_group_colmax(int dt, const void* W, int64_t K, int64_t N, int64_t G, float* s_w,
                               hipStream_t stream);
// Wq (N x K) with the per-group column scales
hipError_t launch_quantize_weight_groups(int dt, const void* W, int64_t K, int64_t N, const float* s_w, int64_t G,
                                         int8_t* Wq, hipStream_t stream);
// Xq (M x K), s_x (M x ng) and rg (ng x M, RN32(s_x/127), group-major) of X's row groups
hipError_t launch_group_xpass(int dt, const void* X, int64_t M, int64_t K, int64_t G, int8_t* Xq, float* s_x,
                              float* rg, hipStream_t stream);
// Y (M x N, 16-bit) = the group-wise product (per-group int32 partials folded into fp32)
hipError_t launch_gemm_group(int dt, const int8_t* Xq, const float* rg, const int8_t* Wq, const float* s_w, int64_t M,
                             int64_t N, int64_t K, int64_t G, void* Y, hipStream_t stream);
// Small batches of the group-wise path (M <= 64, K / G <= 64, where small_batch holds):
// the split-N group kernel.
bool group_small_batch(int64_t M, int64_t K, int64_t N, int64_t G);
hipError_t launch_gemm_group_small(int dt, const int8_t* Xq, const float* rg, const int8_t* Wq, const float* s_w,
                                   int64_t M, int64_t N, int64_t K, int64_t G, void* Y, hipStream_t stream);

}  // namespace llmint8
