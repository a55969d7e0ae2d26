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
// (also zeroes zero[0, n_zero): the product kernel's stream-K tile counters)
hipError_t launch_compact(int64_t M, int64_t K, const uint32_t* partial, uint32_t* bitmap, int32_t* O,
                          int32_t* n_out, hipStream_t stream, int32_t* zero = nullptr, int64_t n_zero = 0);

// The tiled path's stream-K grid (the small-batch routing below consults it).
constexpr int64_t kStreamKGrid = 256;
inline int64_t gemm_tiles(int64_t M, int64_t N) { return ((M + 255) / 256) * ((N + 255) / 256); }
// Workgroups per tile of the stream-K split, by the tile's K stages nk.  A tile's last
// contributor loads and adds the others' partial sums, so a short K loop is better split
// over fewer, longer ranges, some compute units left idle.  Measured on whole calls (cold,
// interleaved on one box) with caps of 2, 3, 4, 6 and 8 against the full grid: nk = 32
// takes 2 (256 x 4096 x 4096: 166 us with the full grid, 60 us; 3 is within 2 us either
// way), nk = 64 takes 3 (4 was 11 us slower on 512 x 8192 x 8192), and longer loops 6
// (128 x 16384 x 8192: 86.3 -> 83.0 us against 3; 256 x 28672 x 8192: 130.9 -> 124.8 us,
// 384 x 16384 x 4096: 98.7 -> 88.0 us against 4).
inline int64_t stream_k_per_tile(int64_t nk) {
    if (nk <= 48) return 2;
    if (nk <= 96) return 3;
    return 6;
}
// the stream-K grid: at most kStreamKGrid workgroups (or the compute units, `cus`, if
// fewer), one per unit (tile and K stage of 128), stream_k_per_tile per tile.  At least
// 2 per tile or half the tiles, so a workgroup's range meets at most three tiles.
inline int64_t stream_k_grid(int64_t M, int64_t K, int64_t N, int64_t cus = kStreamKGrid) {
    const int64_t nk = (K + 127) / 128, T = gemm_tiles(M, N), units = T * nk;
    int64_t g = cus < kStreamKGrid ? cus : kStreamKGrid;
    if (units < g) g = units;
    const int64_t cap = stream_k_per_tile(nk) * T;
    return cap < g ? cap : g;
}
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
    if (N * (1000 + c * M) < 52500000 * (rounds > 0 ? rounds : 1)) return true;
    // Past 64 rows the tiled path runs the stream-K split; on a narrow weight its grid fills
    // less than half the compute units, and while X is small (under 2^20 elements: every
    // workgroup of the small-batch path re-reads all its codes) the small-batch path is
    // faster.  Whole calls, cold, interleaved on one box, small against tiled, N = 8192:
    // 112 x 4096 43.8 / 60.6 us, 128 x 4096 46.8 / 53.0, 112 x 8192 62.6 / 67.8, but
    // 128 x 8192 67.6 / 62.3 (tiled); 128 x 2064 x 7424 34.8 / 48.7; at K = 16384, or at
    // N = 16384 (a grid of 128 or more), the tiled path is as fast or faster.
    return M > 64 && M * K < (int64_t)1 << 20 && 2 * stream_k_grid(M, K, N) < kStreamKGrid;
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
    int8_t* Xqb;  // nullable: the blocked copy of Xq (small batches)
    float* s_x;
    void* XO;
    int64_t xo_pitch;
    const int8_t* Wq;  // NULL: no W_O gather
    void* WO;
};
hipError_t launch_code_rows(const XPassArgs& a, const uint32_t* bitmap, int32_t* O, int32_t* n_out,
                            hipStream_t stream);
// The small-batch X pass also writes Xq in the product kernel's 1 KB blocks (xqb_offset)
// from 8 rows up: with fewer rows the operand loads touch few cache lines either way (at
// M = 1 every lane reads the same row), and the extra writes cost more than they save.
inline bool small_blocked_codes(int64_t M) { return M >= 8; }
// pmax (M x ceil(K/512) words of scratch): per row and 512-column slab, the slab's
// maximum over its non-outlier columns.  with_wo: the tiled product follows, so the coding
// launch also gathers W_O (a.Wq, a.N into a.WO) and zeroes zero[0, n_zero) (the stream-K
// tile counters); the one-workgroup form is not taken then.
hipError_t launch_xpass_small(const XPassArgs& a, int32_t* O, int32_t* n_out, uint32_t* bitmap, uint32_t* pmax,
                              bool with_wo, int32_t* zero, int64_t n_zero, hipStream_t stream);
// The slab X pass also serves the tiled path for few rows (it needs every row of a slab in
// one workgroup), where the detection and the row coding leave most of the device idle.
// Whole steps, cold, interleaved on one box, row path against slab pass: 12288 x 36864 at
// 24, 32, 48, 80, 96 and 112 rows 127.6 / 124.4, 128.5 / 124.2, 136.6 / 131.1, 141.9 /
// 138.9, 142.6 / 139.5 and 149.5 / 145.8 us; 4096 x 16384 at 80, 96 and 112 rows 59.3 /
// 57.4, 60.5 / 58.0 and 62.7 / 59.4 us; 28672 x 8192 at 112 rows 120.0 / 117.2 us.  At 128
// rows the row path was 1.6 to 2.5 us faster on all three weights.
constexpr int64_t kSlabXPassM = 112;
inline bool slab_xpass(int64_t M, int64_t K) { return M > 0 && M <= kSlabXPassM && K <= kSmallK; }

// ---- products + epilogue
struct GemmArgs {
    int dt;
    const int8_t* Xq;
    int64_t xq_pitch;
    const int8_t* Xqb = nullptr;  // small-batch kernel: the blocked copy of Xq when the X
                                  // pass wrote one (xqb_offset), else Xq row by row
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
    int32_t* sk_cnt = nullptr;   // stream-K tile counters (zero between calls) and partial
    int32_t* sk_part = nullptr;  // slots, when the workspace holds them (stream_k_shape)
};
// Stream-K on the tiled path: with fewer tiles than twice the grid (kStreamKGrid at most,
// one workgroup per compute unit) and not a multiple of it, the tiles' K stages are split
// evenly over the grid.  The workspace then holds one counter per tile and two 256 x 256
// int32 partial tiles per workgroup.
inline bool stream_k_shape(int64_t M, int64_t K, int64_t N) {
    const int64_t T = gemm_tiles(M, N);
    return M > 0 && N > 0 && K > 0 && !small_batch(M, K, N) && T < 2 * kStreamKGrid && T % kStreamKGrid != 0;
}
constexpr int64_t kStreamKSlotBytes = 256 * 256 * 4;
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
// Xq (M x K), s_x (M x ng) and rg (ng x M, RN32(s_x/127), group-major) of X's row groups,
// and, when Xqb is not NULL, Xq again in the small-batch kernel's 1 KB blocks (xqb_offset)
hipError_t launch_group_xpass(int dt, const void* X, int64_t M, int64_t K, int64_t G, int8_t* Xq, float* s_x,
                              float* rg, int8_t* Xqb, hipStream_t stream);
// Y (M x N, 16-bit) = the group-wise product (per-group int32 partials folded into fp32)
hipError_t launch_gemm_group(int dt, const int8_t* Xq, const float* rg, const int8_t* Wq, const float* s_w, int64_t M,
                             int64_t N, int64_t K, int64_t G, void* Y, hipStream_t stream);
// Small batches of the group-wise path (M <= 64, K / G <= 64, where small_batch holds):
// the split-N group kernel, reading the blocked copy Xqb when it is not NULL.
bool group_small_batch(int64_t M, int64_t K, int64_t N, int64_t G);
// The part of group_small_batch that does not depend on N, with at least 8 rows and groups
// of 256 to 1024: where the group X pass writes the blocked copy (it runs before N is
// known).
bool group_blocked_codes(int64_t M, int64_t K, int64_t G);
hipError_t launch_gemm_group_small(int dt, const int8_t* Xq, const int8_t* Xqb, const float* rg, const int8_t* Wq,
                                   const float* s_w, int64_t M, int64_t N, int64_t K, int64_t G, void* Y,
                                   hipStream_t stream);

}  // namespace llmint8
