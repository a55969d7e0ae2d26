// The products of the LLM.int8() matmul and its dequantizing epilogue, one kernel:
//   C = Xq Wq^T            int8 x int8 -> int32 on v_mfma_i32_32x32x32_i8 (exact),
//   F = X[:,O] Wq[:,O]^T   16-bit x 16-bit -> fp32 on v_mfma_f32_32x32x16_{f16,bf16},
//   y = RN((RN(RN((float)C * r_i) * c_n)) + RN(c_n * F)),  r_i = s_x/127, c_n = s_w/127
//     (with a fixed outlier set whose W rows are kept in 16 bits: + F, unscaled),
//   Y = y rounded to the 16-bit type.
// "LLM.int8(): 8-bit Matrix Multiplication for Transformers at Scale", abstract: the
// int8 product with one normalization constant per inner-product vector, and the
// outlier feature dimensions through a 16-bit product, summed into the same output.
//
// Tiling (gfx950: 64-wide waves, 160 KB LDS, 512 registers per lane per SIMD):
//   block tile 256 x 256, 8 waves in 2 x 4 -- two per SIMD, 256 registers each --, each
//   wave 128 x 64 = 4 x 2 MFMA tiles of 32 x 32 -> 128 int32 accumulators per lane.  With
//   two waves on a SIMD, one wave's MFMAs keep the matrix unit busy while the other waits
//   at a barrier or for its operands (one wave of 128 x 128 per SIMD left it idle there);
//   the LDS, which then serves 0.75 KB per MFMA instead of 0.5, has the bandwidth for it.
//   (On gfx950 the 32x32x32 i8 MFMA sustains the full int8 rate; the 16x16x64 form issues
//   at about half of it.)
//   Operands go HBM/L2 -> LDS with buffer loads straight into LDS (16 B per lane, no
//   register staging; a buffer resource per operand over the tile's rows, so a load sends
//   32-bit offsets and the stage's K position rides in the scalar offset), one 128-byte
//   line per row per K stage (full-line requests).  The LDS
//   holds 2 A slots and 3 B slots of 32 KB: during stage k the loads of A[k+1] and
//   B[k+2] are issued (the weight panels get the longer lead: 1.4 % faster than the
//   other way round on the 4096 x 12288 x 36864 projection, 1.3 % slower on the
//   8192 x 28672 x 8192 one).  Waits are counted
//   (vmcnt) and the workgroup barrier is a bare s_barrier, so a barrier never drains the
//   loads still in flight.  Each stage is four 32-deep MFMA sub-steps; the operands of
//   the next sub-step are read from LDS into a second register set while the 8 MFMAs
//   of the current one run.  The instruction order inside a sub-step (global loads and
//   LDS reads front-loaded between the MFMAs) is pinned with scheduling-group hints, and
//   each sub-step begins with an LDS wait that costs nothing.  The
//   16-byte chunk c of LDS row r sits at chunk c ^ (r & 7) ^ ((r >> 3) & 1), so the
//   ds_read_b128 of 16 consecutive rows at one k hit distinct banks (for both 8- and
//   16-lane service groups).
//   Tiles are assigned so that the workgroups the dispatcher places on one XCD (ids
//   congruent mod 8) take a contiguous run of tiles in grouped order (8 row-tiles per
//   group): the 32 tiles running together on an XCD share A and B panels in its L2.
//   Persistent: one workgroup per compute unit works through its XCD's run, strided by
//   the XCD's workgroup count.  Its K stages run back to back across tile boundaries --
//   the loads of a tile's last stages already fetch the next tile's first operands --,
//   and a tile's epilogue (outlier product, dequantization, Y through the two LDS slots
//   its last stage freed) runs while those are in flight.  Against one workgroup per tile,
//   that removes the pipeline fill (about 2.5 us) and the workgroup launch (about 1.3 us)
//   from every tile boundary.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace llmint8 {

namespace {

constexpr int NJ = 2;                                    // 32-column MFMA tiles per wave along N
constexpr int kWaves = 8;                                // 2 (M) x 4 (N), two per SIMD
constexpr int BM = 256, BN = 4 * 32 * NJ;
constexpr int BK = 128;                                  // bytes of K per stage: one line per row
constexpr int kTileBytes = BM * BK;                      // one operand's stage: 32 KB
constexpr int kChunks = BK / 16;                         // 16-byte chunks per row segment
constexpr int kRowsPerLoad = 64 / kChunks;               // rows covered by one 64-lane load
constexpr int kLoadsA = BM / kRowsPerLoad / kWaves;      // per wave, per stage (4)
constexpr int kLoadsB = BN / kRowsPerLoad / kWaves;      // per wave, per stage (4)
constexpr bool kLeadA = false;                           // which operand is loaded two stages ahead
constexpr int kSlotsA = kLeadA ? 3 : 2;                  // 5 x 32 KB: the whole 160 KB of LDS
constexpr int kSlotsB = kLeadA ? 2 : 3;
constexpr int kSlotBytesB = BN * BK;
constexpr int kSubSteps = BK / 32;                       // 32-deep MFMA steps per stage
constexpr int kGroupM = 8;                               // row tiles per group of the tile order
// epilogue staging, in the A and B slots the tile's last stage freed: the tile's row and
// column factors, then per wave one 32 x 64 slice of its outputs at a time, rows padded to
// 144 bytes (16-byte aligned)
constexpr int kScaleBytes = 2 * 256 * 4;
constexpr int kYPitch = 72;  // 16-bit elements
constexpr int kYQuarterBytes = 32 * kYPitch * 2;
constexpr int kXcds = 8;
static_assert(kSlotsA * kTileBytes + kSlotsB * kSlotBytesB <= 160 * 1024, "LDS");
static_assert(kLoadsA == 4 && kLoadsB == 4, "the waits below count 4 loads per operand and wave");
static_assert(kScaleBytes + 4 * kYQuarterBytes <= kTileBytes && 4 * kYQuarterBytes <= kSlotBytesB, "epilogue LDS");
static_assert(!kLeadA && kSlotsA == 2 && kSlotsB == 3, "the stage loop rotates 2 A slots and 3 B slots, B two ahead");
static_assert(BM == 256 && BN == 256, "the factor tables take one row and one column per thread");

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// A raw buffer resource over `bytes` bytes from `base` (dword data format, as gfx9 buffer
// loads expect): loads at offsets past `bytes` return zero and touch no memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, 0x00020000);
}

// 16 bytes per lane from the resource at voffset + soffset into LDS at lds_base + 16 * lane.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rs, uint32_t voffset, int soffset, int8_t* lds_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)lds_base, 16, (int)voffset, soffset, 0, 0);
}

// Chunk swizzle: the 16-byte chunk c of LDS row r is stored at chunk c ^ swz(r), so that
// the ds_read_b128 of 16 consecutive rows at one chunk touch distinct banks.
__host__ __device__ constexpr int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// Wait until this wave's LDS reads are done (a builtin, so the compiler knows) and at most
// N of its direct-to-LDS loads are in flight, then the workgroup barrier (no fence: later
// loads stay in flight).  0xC07F: s_waitcnt lgkmcnt(0) with vmcnt and expcnt unconstrained.
#define LLMINT8_WAIT_BARRIER(N)                                  \
    do {                                                         \
        __builtin_amdgcn_s_waitcnt(0xC07F);                      \
        asm volatile("s_waitcnt vmcnt(" #N ")\n\ts_barrier" ::: "memory"); \
    } while (0)

struct Params {
    const int8_t* Xq;
    int64_t xq_pitch;
    const int8_t* Wq;
    int64_t M, N, K;
    const float* s_x;
    const float* s_w;
    const uint16_t* XO;
    const uint16_t* WO;
    int64_t xo_pitch, wo_pitch;
    int f_scaled;
    const int32_t* n_out;
    uint16_t* Y;
    int32_t* C_acc;
    float* F_acc;
    int tiles_m, tiles_n;
    int32_t* sk_cnt;   // stream-K: per tile, the contributors done so far (0 between calls)
    int32_t* sk_part;  // stream-K: two 256 x 256 int32 partial tiles per workgroup
};

template <int DT>
__device__ __forceinline__ v16f mfma16(const u32x4& a, const u32x4& b, const v16f& c) {
    if constexpr (DT == F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, a), __builtin_bit_cast(v8h, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
}

// SK (stream-K, for calls with fewer tiles than twice the workgroups, not a multiple of
// them): the K stages of all tiles, taken in order (tile t's stages are units t nk .. t nk +
// nk - 1), are split evenly over the workgroups; a workgroup's range covers at most three
// segments of tiles.  A segment that is a whole tile ends in the epilogue as usual.  A part
// of a tile ends by storing its exact int32 partial sums to the workgroup's slot and
// counting itself in on the tile's counter; the tile's last contributor adds the others'
// partials (integer sums: the order does not matter) and runs the epilogue, so Y is the
// same bits as without the split.  It leaves the counter at 0 again (the X pass zeroes the
// counters; every call leaves them so).
// HALF (M <= 128: every valid row lies in the first half of its tile): the four waves of
// rows 128..255 issue their share of the loads and meet every barrier, but run no MFMA and
// read no operands, so each SIMD's matrix unit serves one wave.
template <int DT, bool ACC_OUT, bool SK, bool HALF>
__global__ __launch_bounds__(64 * kWaves) void gemm_kernel(Params p) {
    __shared__ __attribute__((aligned(1024))) int8_t smem[kSlotsA * kTileBytes + kSlotsB * kSlotBytesB];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w >> 2, wn = w & 3;
    const int nk = (int)ceil_div(p.K, BK);  // >= 1 (K = 0 never reaches this kernel)

    // ---- tiles of this workgroup: the XCD-contiguous run of tiles (grouped order) of the
    // XCD the dispatcher places it on (ids congruent mod 8), strided by the number of
    // workgroups on that XCD (SK: the segments of its range of units)
    const int T = p.tiles_m * p.tiles_n;
    const int bid = blockIdx.x, nwg = gridDim.x;
    const int xcd = bid % kXcds, local = bid / kXcds;
    const int per = T / kXcds, rem = T % kXcds;
    const int x_start = xcd * per + (xcd < rem ? xcd : rem), x_cnt = per + (xcd < rem ? 1 : 0);
    const int on_xcd = (nwg - xcd + kXcds - 1) / kXcds;
    const int64_t sk_units = (int64_t)T * nk;
    auto sk_begin = [&](int c) -> int64_t { return sk_units * c / nwg; };
    // segments s = 0, 1, 2: tile t_s, first stage k_s, stages n_s (scalars, not an array: an
    // array indexed by the segment number would live in scratch memory)
    int t_0 = 0, t_1 = 0, t_2 = 0, k_0 = 0, k_1 = 0, k_2 = 0, n_0 = nk, n_1 = nk, n_2 = nk;
    int my_tiles = 0;
    if constexpr (SK) {
        int64_t u = sk_begin(bid);
        const int64_t u1 = sk_begin(bid + 1);
        // past the range: whole-tile dummies (tile 0, all stages), loaded through empty resources
        auto next = [&](int& t, int& k, int& n) {
            if (u < u1) {
                t = (int)(u / nk);
                const int64_t e = (int64_t)(t + 1) * nk < u1 ? (int64_t)(t + 1) * nk : u1;
                k = (int)(u - (int64_t)t * nk);
                n = (int)(e - u);
                ++my_tiles;
                u = e;
            }
            t = __builtin_amdgcn_readfirstlane(t);  // uniform: scalar registers
            k = __builtin_amdgcn_readfirstlane(k);
            n = __builtin_amdgcn_readfirstlane(n);
        };
        next(t_0, k_0, n_0);
        next(t_1, k_1, n_1);
        next(t_2, k_2, n_2);
        my_tiles = __builtin_amdgcn_readfirstlane(my_tiles);
    } else {
        my_tiles = local < x_cnt ? (x_cnt - local + on_xcd - 1) / on_xcd : 0;
    }
    if (my_tiles == 0) return;  // the same for every wave of the workgroup
    auto seg_tile = [&](int i) { return i <= 0 ? t_0 : (i == 1 ? t_1 : t_2); };
    auto seg_k = [&](int i) { return i <= 0 ? k_0 : (i == 1 ? k_1 : k_2); };
    auto seg_n = [&](int i) { return i <= 0 ? n_0 : (i == 1 ? n_1 : n_2); };
    auto tile_origin = [&](int i, int64_t& m0, int64_t& n0) {
        if constexpr (SK) {
            const int t = seg_tile(i);
            m0 = (int64_t)(t % p.tiles_m) * BM;
            n0 = (int64_t)(t / p.tiles_m) * BN;
        } else {
            const int t = x_start + local + i * on_xcd;
            const int in_group = kGroupM * p.tiles_n;
            const int first_m = (t / in_group) * kGroupM;
            const int gm = p.tiles_m - first_m < kGroupM ? p.tiles_m - first_m : kGroupM;
            m0 = (int64_t)(first_m + (t % in_group) % gm) * BM;
            n0 = (int64_t)((t % in_group) / gm) * BN;
        }
    };

    // ---- per-lane offsets of the stage loop: loader (wave w fills LDS slots
    // [1024*(4w+j), +1024) of each operand, j = 0..3: row r = 8*(4w + j) + lane/8 of the
    // tile, one 128-byte line per row, physical chunk lane%8, logical chunk
    // (lane%8) ^ swz(r)) and MFMA operand reads (32x32x32: lane holds row lane%32, 16 k at
    // 16*(lane/32); fragment i of sub-step u reads row 32*i + lane%32 of the wave's
    // 128-row panel, logical chunk 2u + lane/32).  They are recomputed after every
    // epilogue from an opaque copy of the lane index, so that they are not held through it.
    const int wu = __builtin_amdgcn_readfirstlane(w);
    uint32_t a_off[kLoadsA], b_off[kLoadsB];
    int rd[kSubSteps];
    auto lane_offsets = [&](int ln) {
#pragma unroll
        for (int j = 0; j < kLoadsA; ++j) {
            const int r = kRowsPerLoad * (kLoadsA * wu + j) + ln / kChunks;
            a_off[j] = (uint32_t)(r * p.xq_pitch + (((ln % kChunks) ^ swz(r)) << 4));
        }
#pragma unroll
        for (int j = 0; j < kLoadsB; ++j) {
            const int r = kRowsPerLoad * (kLoadsB * wu + j) + ln / kChunks;
            b_off[j] = (uint32_t)(r * p.K + (((ln % kChunks) ^ swz(r)) << 4));
        }
        const int rl = ln & 31, h = ln >> 5;
#pragma unroll
        for (int u = 0; u < kSubSteps; ++u) rd[u] = rl * BK + (((2 * u + h) ^ swz(rl)) << 4);
    };
    lane_offsets(lane);

    // ---- operand resources.  A tile's resources span its rows (at most 256 of them:
    // offsets fit 32 bits for any K the library accepts); rows past M or N lie past the
    // resource and read zero.  In a partial last stage the chunks past K of a B row read
    // the next row's first bytes, or nothing (zero) past the last row: their A side is the
    // zero padding of Xq, so they add exact zeros.  Loads run up to two stages ahead, across
    // tile boundaries: the resources of this tile and the next two are held.  Past the
    // workgroup's last tile a resource is empty: every stage issues its loads, and those
    // land zeros in slots no stage reads.
    auto tile_rsrc = [&](int i, __amdgpu_buffer_rsrc_t& ra, __amdgpu_buffer_rsrc_t& rb) {
        int64_t m0 = 0, n0 = 0, rows_a = 0, rows_b = 0;
        if (i < my_tiles) {
            tile_origin(i, m0, n0);
            rows_a = p.M - m0 < BM ? p.M - m0 : BM;
            rows_b = p.N - n0 < BN ? p.N - n0 : BN;
        }
        ra = buffer_rsrc(p.Xq + m0 * p.xq_pitch, rows_a * p.xq_pitch);
        rb = buffer_rsrc(p.Wq + n0 * p.K, rows_b * p.K);
    };
    __amdgpu_buffer_rsrc_t ra0, rb0, ra1, rb1, ra2, rb2;
    tile_rsrc(0, ra0, rb0);
    tile_rsrc(1, ra1, rb1);
    tile_rsrc(2, ra2, rb2);

    // The workgroup's stages run back to back over its tiles: global stage s sits in A slot
    // s % 2 and B slot s % 3.  `d` = tiles ahead of the current one.
    auto slot_a = [&](int sa) { return smem + sa * kTileBytes; };
    auto slot_b = [&](int sb) { return smem + kSlotsA * kTileBytes + sb * kSlotBytesB; };
    auto issue_a = [&](int sa, int kt, int d) {
        const __amdgpu_buffer_rsrc_t rs = d == 0 ? ra0 : (d == 1 ? ra1 : ra2);
        int8_t* As = slot_a(sa);
#pragma unroll
        for (int j = 0; j < kLoadsA; ++j) load_lds16(rs, a_off[j], kt * BK, As + (kLoadsA * wu + j) * 1024);
    };
    auto issue_b = [&](int sb, int kt, int d) {
        const __amdgpu_buffer_rsrc_t rs = d == 0 ? rb0 : (d == 1 ? rb1 : rb2);
        int8_t* Bs = slot_b(sb);
#pragma unroll
        for (int j = 0; j < kLoadsB; ++j) load_lds16(rs, b_off[j], kt * BK, Bs + (kLoadsB * wu + j) * 1024);
    };
    auto read_frags = [&](int sa, int sb, int u, v4i (&fa)[4], v4i (&fb)[NJ]) {
        const int8_t* As = slot_a(sa) + wm * 128 * BK + rd[u];
        const int8_t* Bs = slot_b(sb) + wn * (32 * NJ) * BK + rd[u];
        fa[0] = *(const v4i*)As;
#pragma unroll
        for (int j = 0; j < NJ; ++j) fb[j] = *(const v4i*)(Bs + j * 32 * BK);
#pragma unroll
        for (int i = 1; i < 4; ++i) fa[i] = *(const v4i*)(As + i * 32 * BK);
    };

    v16i acc[4][NJ];
    auto mfma_rows = [&](const v4i (&fa)[4], const v4i (&fb)[NJ], int i0, int i1) {
#pragma unroll
        for (int i = i0; i < i1; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
    };

    // ---- the epilogue's global reads, issued in a tile's last stage (whose closing wait
    // then covers them): this thread's entry of the factor tables (waves 0-3: the rows'
    // s_x, waves 4-7: the columns' s_w) at its top, and the first 16 outlier columns of the
    // wave's rows and columns after its barrier (in the registers the next stage's first
    // operands take elsewhere).  Unconditional buffer loads: with no outlier column the
    // resources are empty and the loads return zeros.
    const int32_t nO = *p.n_out;
    const int nsub = (nO + 15) >> 4;  // 16-deep MFMA steps over the padded outlier columns
    float sc = 0.0f;
    u32x4 xo0[4], wo0[NJ];
    auto epilogue_reads = [&](int ti, bool outlier_part) {
        int lx = lane, tx = tid;
        asm volatile("" : "+v"(lx), "+v"(tx));
        const int rl = lx & 31, h = lx >> 5, tid = tx;
        const int w = __builtin_amdgcn_readfirstlane(tx >> 6), wm = w >> 2, wn = w & 3;
        int64_t m0, n0;
        tile_origin(ti, m0, n0);
        if (outlier_part) {
            const int64_t rows = nsub > 0 ? (p.M - m0 < BM ? p.M - m0 : BM) : 0;
            const __amdgpu_buffer_rsrc_t rx = buffer_rsrc(p.XO + m0 * p.xo_pitch, rows * p.xo_pitch * 2);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                xo0[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                       rx, (uint32_t)(((wm * 128 + 32 * i + rl) * p.xo_pitch + h * 8) * 2), 0, 0));
        } else {
            const int64_t cols = nsub > 0 ? (p.N - n0 < BN ? p.N - n0 : BN) : 0;
            const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(p.WO + n0 * p.wo_pitch, cols * p.wo_pitch * 2);
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                wo0[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                       rw, (uint32_t)(((wn * (32 * NJ) + 32 * j + rl) * p.wo_pitch + h * 8) * 2), 0, 0));
            // factor tables: rows m0 + tid (waves 0-3) or columns n0 + tid - 256 (waves 4-7)
            const bool rows_side = w < 4;
            const int64_t base = rows_side ? m0 : n0, lim = rows_side ? p.M : p.N;
            const int64_t cnt = lim - base < BM ? lim - base : BM;
            const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(rows_side ? (const void*)(p.s_x + m0) : (const void*)(p.s_w + n0), cnt * 4);
            sc = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, (uint32_t)((tid & (BM - 1)) * 4), 0, 0));
        }
    };

    // One K stage (global stage s in slots sa, sb; stage kt of its tile).  Sub-steps 0..2
    // run their 8 MFMAs while the 6 LDS reads of the next sub-step (and, in 0 and 1, the
    // global loads of stage s+1 of the short-lead operand and stage s+2 of the long-lead
    // one, into the slots stage s-1 freed) are interleaved, front-loaded so they have most
    // of the sub-step to land.  Sub-step 3 runs 2 MFMAs, waits for stage s+1 and meets the
    // other waves at the barrier, then reads stage s+1's first operands under its other 6
    // -- except in a tile's last stage (LAST), where the epilogue comes first.  Each
    // sub-step is fenced (sched_barrier) so that the interleave stays inside it.
    v4i fa[2][4], fb[2][NJ];  // operand sets of the current / next sub-step
    // where the loads of stage kt of segment ti go: stage ka of tile d_a ahead (A), stage
    // kb of tile d_b ahead (B)
    auto stage_loads = [&](int kt, int ti, int& ka, int& da, int& kb, int& db) {
        // (readfirstlane: the compiler then knows these, and so the resources, are uniform)
        if constexpr (SK) {
            // kt counts this segment's stages; the loads take absolute stages (the segment's
            // first stage + its count), running on into the next segments
            const int l0 = seg_n(ti), l1 = seg_n(ti + 1);
            da = __builtin_amdgcn_readfirstlane(kt + 1 < l0 ? 0 : 1);
            ka = __builtin_amdgcn_readfirstlane(da == 0 ? seg_k(ti) + kt + 1 : seg_k(ti + 1) + kt + 1 - l0);
            db = __builtin_amdgcn_readfirstlane(kt + 2 < l0 ? 0 : (kt + 2 - l0 < l1 ? 1 : 2));
            kb = __builtin_amdgcn_readfirstlane(
                db == 0 ? seg_k(ti) + kt + 2
                        : (db == 1 ? seg_k(ti + 1) + kt + 2 - l0 : seg_k(ti + 2) + kt + 2 - l0 - l1));
        } else {
            ka = kt + 1 < nk ? kt + 1 : kt + 1 - nk;
            da = __builtin_amdgcn_readfirstlane(kt + 1 < nk ? 0 : 1);
            db = __builtin_amdgcn_readfirstlane(kt + 2 < nk ? 0 : (kt + 2 < 2 * nk ? 1 : 2));
            kb = kt + 2 - db * nk;
        }
    };
    auto stage = [&](int sa, int sb, int kt, int ti, auto last_tag) {
        constexpr bool LAST = decltype(last_tag)::value;
        int ka, da, kb, db;
        stage_loads(kt, ti, ka, da, kb, db);
        if constexpr (LAST && !ACC_OUT) {
            epilogue_reads(ti, false);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int u = 0; u < kSubSteps - 1; ++u) {
            const int cur = u & 1, nxt = cur ^ 1;
            // this sub-step's operands were read a sub-step ago: a free wait that keeps the
            // compiler's own waits (it counts the direct-to-LDS loads as LDS traffic) out
            __builtin_amdgcn_s_waitcnt(0xC07F);
            if (u == 0) issue_a(sa ^ 1, ka, da);
            if (u == 1) issue_b(sb == 0 ? 2 : sb - 1, kb, db);
            read_frags(sa, sb, u + 1, fa[nxt], fb[nxt]);
            mfma_rows(fa[cur], fb[cur], 0, 4);
            if (u < 2) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                }
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                }
            } else {
#pragma unroll
                for (int q = 0; q < 6; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                }
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        mfma_rows(fa[1], fb[1], 0, 1);
        __builtin_amdgcn_sched_barrier(0);
        LLMINT8_WAIT_BARRIER(4);  // the stage s+2 loads may stay in flight
        if constexpr (!LAST) read_frags(sa ^ 1, sb == 2 ? 0 : sb + 1, 0, fa[0], fb[0]);
        else if constexpr (!ACC_OUT) epilogue_reads(ti, true);
        mfma_rows(fa[1], fb[1], 1, 4);
        __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
        __builtin_amdgcn_sched_barrier(0);
    };

    // HALF, rows 128..255: the stage's loads and its barrier, no operand reads or products
    auto idle_stage = [&](int sa, int sb, int kt, int ti, auto last_tag) {
        constexpr bool LAST = decltype(last_tag)::value;
        int ka, da, kb, db;
        stage_loads(kt, ti, ka, da, kb, db);
        if constexpr (LAST && !ACC_OUT) epilogue_reads(ti, false);  // the column factors
        issue_a(sa ^ 1, ka, da);
        issue_b(sb == 0 ? 2 : sb - 1, kb, db);
        LLMINT8_WAIT_BARRIER(4);
    };

    // ---- epilogue of tile ti: 16-bit outlier product, dequantization, Y.  The LDS slots of
    // the stage just consumed (A sa, B sb) are free: no wave reads them past that stage's
    // barrier, and the loads in flight go to the other slots.
    auto epilogue = [&](int ti, int sa, int sb) {
        // lane-derived values made opaque here, so that the compiler computes the
        // epilogue's addresses in it instead of holding them through the main loop
        int lx = lane, tx = tid;
        asm volatile("" : "+v"(lx), "+v"(tx));
        const int rl = lx & 31, h = lx >> 5, lane = lx, tid = tx;
        const int w = __builtin_amdgcn_readfirstlane(tx >> 6), wm = w >> 2, wn = w & 3;
        int64_t m0, n0;
        tile_origin(ti, m0, n0);
        const int64_t wm0 = m0 + wm * 128, wn0 = n0 + wn * (32 * NJ);
        if constexpr (ACC_OUT) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t row0 = wm0 + 32 * i + 4 * h;
                int64_t am = wm0 + 32 * i + rl;
                am = am < p.M ? am : p.M - 1;
                const uint16_t* xo = p.XO + am * p.xo_pitch + h * 8;
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const int64_t n = wn0 + 32 * j + rl;
                    const int64_t bn = n < p.N ? n : p.N - 1;
                    const uint16_t* wo = p.WO + bn * p.wo_pitch + h * 8;
                    v16f F = v16f{};
                    for (int ch = 0; ch < nsub; ++ch)
                        F = mfma16<DT>(*(const u32x4*)(xo + ch * 16), *(const u32x4*)(wo + ch * 16), F);
                    if (n >= p.N) continue;
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int64_t m = row0 + 8 * (e >> 2) + (e & 3);
                        if (m >= p.M) continue;
                        p.C_acc[m * p.N + n] = acc[i][j][e];
                        p.F_acc[m * p.N + n] = F[e];
                    }
                }
            }
        } else {
            float* rsc = (float*)slot_a(sa);  // r_i = s_x[i]/127 of the tile's rows
            float* csc = rsc + BM;            // c_n = s_w[n]/127 of its columns
            rsc[tid] = sc / 127.0f;           // (csc[tid - 256] for waves 4-7)
            __builtin_amdgcn_s_waitcnt(0xC07F);
            __builtin_amdgcn_s_barrier();
            // per wave, a 32 x 64 staging area (rows padded to 144 bytes): waves 0-3 in the
            // free A slot after the factor tables, waves 4-7 in the free B slot
            uint16_t* ys = (uint16_t*)(w < 4 ? slot_a(sa) + kScaleBytes + w * kYQuarterBytes
                                             : slot_b(sb) + (w - 4) * kYQuarterBytes);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rb = wm * 128 + 32 * i + 4 * h;  // tile row of e = 0
                // the slice's 16-bit outlier products: the first 16 columns from the
                // prefetched operands, the rest one 16-column step (both column tiles) per
                // round trip
                v16f F[NJ];
#pragma unroll
                for (int j = 0; j < NJ; ++j) F[j] = mfma16<DT>(xo0[i], wo0[j], v16f{});
                if (nsub > 1) {
                    int64_t am = wm0 + 32 * i + rl;
                    am = am < p.M ? am : p.M - 1;
                    const uint16_t* xo = p.XO + am * p.xo_pitch + h * 8;
                    const uint16_t* wo[NJ];
#pragma unroll
                    for (int j = 0; j < NJ; ++j) {
                        const int64_t n = wn0 + 32 * j + rl;
                        wo[j] = p.WO + (n < p.N ? n : p.N - 1) * p.wo_pitch + h * 8;
                    }
                    for (int ch = 1; ch < nsub; ++ch) {
                        const u32x4 xa = *(const u32x4*)(xo + ch * 16);
                        u32x4 wa[NJ];
#pragma unroll
                        for (int j = 0; j < NJ; ++j) wa[j] = *(const u32x4*)(wo[j] + ch * 16);
#pragma unroll
                        for (int j = 0; j < NJ; ++j) F[j] = mfma16<DT>(xa, wa[j], F[j]);
                    }
                }
                // the columns' factors, and the slice's row factors four at a time (one table
                // read for both column tiles): read between the staging stores one by one,
                // each would be read again and waited for before every element, since the
                // compiler cannot tell the table from the staging area
                float c[NJ], cf[NJ];
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    c[j] = csc[wn * (32 * NJ) + 32 * j + rl];
                    // the outlier term's factor: c_n, or 1 (an exact product) when W_O holds
                    // 16-bit rows of W
                    cf[j] = p.f_scaled ? c[j] : 1.0f;
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const v4f rf = *(const v4f*)(rsc + rb + 8 * q);
#pragma unroll
                    for (int j = 0; j < NJ; ++j)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int e = 4 * q + r;
                            const float yi = __fmul_rn(__fmul_rn((float)acc[i][j][e], rf[r]), c[j]);
                            const float y = __fadd_rn(yi, __fmul_rn(cf[j], F[j][e]));
                            ys[(8 * q + 4 * h + r) * kYPitch + 32 * j + rl] = from_f32<DT>(y);
                        }
                }
                // all the prefetched outlier operands are in before the first stores (else
                // the compiler's wait for a later slice's would also wait for the stores)
                if (i == 0) asm volatile("" ::"v"(xo0[1]), "v"(xo0[2]), "v"(xo0[3]));
                // read the slice back as 16-byte row segments (one wave's LDS accesses
                // complete in order) and store them (full lines)
#pragma unroll
                for (int it = 0; it < 4; ++it) {
                    const int row = it * 8 + (lane >> 3), ch = lane & 7;
                    const u32x4 v = *(const u32x4*)(ys + row * kYPitch + ch * 8);
                    const int64_t m = wm0 + 32 * i + row, n = wn0 + ch * 8;
                    if (m < p.M && n < p.N) *(u32x4*)(p.Y + m * p.N + n) = v;
                }
            }
        }
    };

    // ---- stream-K: the end of a segment that is part of a tile (see the kernel's comment).
    // The partial sums go to slot 2 bid + (first segment of the range ? 0 : 1), 16-byte
    // piece (accumulator quarter) * 512 + tid; the partial parts of a tile are the first or
    // the last segment of their workgroups' ranges.  Slots and counters are written and read
    // with the agent-scope coherence bit, coherent across the XCDs without writing back or
    // invalidating any L2 (that would cost the other workgroups their operands).
    // (the grid has at most one workgroup per unit: every range holds at least one unit)
    auto sk_owner = [&](int64_t x) {  // the workgroup whose range holds unit x
        int c = (int)(x * nwg / sk_units);
        while (c > 0 && sk_begin(c) > x) --c;
        while (c + 1 < nwg && sk_begin(c + 1) <= x) ++c;
        return c;
    };
    auto sk_slot = [&](int c, int t) {
        return p.sk_part + (int64_t)(2 * c + (sk_begin(c) / nk == t ? 0 : 1)) * (BM * BN);
    };
    // (the verdict travels through the last word of the B slot the segment's last stage
    // freed: the epilogue's staging stops short of it and no load in flight goes there)
    static_assert(4 * kYQuarterBytes + 4 <= kSlotBytesB, "stream-K flag");
    auto sk_finish = [&](int ti, int sa, int sb) -> bool {  // true: this workgroup runs the tile's epilogue
        int* sk_flag = (int*)(slot_b(sb) + kSlotBytesB - 4);
        const int t = seg_tile(ti);
        if (seg_k(ti) == 0 && seg_n(ti) == nk) return true;
        // the 32 x 32 blocks of the wave that hold outputs (a mid-size batch fills a
        // quarter of the rows), 16 bytes per lane, through a buffer resource over the slot
        // with the agent-scope coherence bit (sc1, cache policy 16): coherent across XCDs
        int64_t m0, n0;
        tile_origin(ti, m0, n0);
        const int64_t vr = p.M - m0, vc = p.N - n0;  // valid rows / columns of the tile
        auto block_live = [&](int i, int j) {
            return (int64_t)(wm * 128 + 32 * i) < vr && (int64_t)(wn * (32 * NJ) + 32 * j) < vc;
        };
        constexpr int kCoherent = 16;
        auto slot_rsrc = [&](int c) { return buffer_rsrc(sk_slot(c, t), (int64_t)BM * BN * 4); };
        // lane part in the one VGPR offset, piece part in the scalar offset (a VGPR per
        // piece would be hoisted over the main loop)
        const uint32_t lane_off = (uint32_t)tid * 16;
        auto piece = [&](int i, int j, int q) { return (uint32_t)(((i * NJ + j) * 4 + q) * (64 * kWaves) * 16); };
        {
            const __amdgpu_buffer_rsrc_t rs = slot_rsrc(bid);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    if (block_live(i, j))
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            __builtin_amdgcn_raw_buffer_store_b128(
                                __builtin_bit_cast(u32x4, v4i{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                                              acc[i][j][4 * q + 3]}),
                                rs, lane_off, piece(i, j, q), kCoherent);
        }
        // every wave's stores complete before the count
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        if (tid == 0) {
            const int c0 = sk_owner((int64_t)t * nk), c1 = sk_owner((int64_t)(t + 1) * nk - 1);
            const int done = __hip_atomic_fetch_add(&p.sk_cnt[t], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1;
            *sk_flag = done == c1 - c0 + 1 ? 1 : 0;
            if (*sk_flag) __hip_atomic_store(&p.sk_cnt[t], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_s_barrier();
        const int last = __builtin_amdgcn_readfirstlane(*sk_flag);
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_s_barrier();  // every wave has the verdict before the slot is reused
        if (!last) return false;
        // the last contributor: the others' partials (complete before they counted in).  They
        // come through the two LDS slots the last stage freed (A slot sa, B slot sb; the
        // verdict above is read, so its word may go): a wave's live pieces of kRows rows of
        // 32 x 32 blocks are loaded straight into its own region of them with the coherence
        // bit, all in flight at once (they hold no registers), then read back and added.
        // Loaded into registers instead, one 16-byte piece was in flight at a time (the
        // accumulators leave four registers free here): 32 dependent round trips per
        // partial.  The half-tile mode's four output waves take two rows a round, 16 KB each.
        constexpr int kRows = HALF ? 2 : 1;
        constexpr int kRegion = kRows * NJ * 4 * 1024;  // bytes per wave and round
        constexpr int kPerSlot = kTileBytes / kRegion;    // waves per slot
        static_assert(kTileBytes == kSlotBytesB && kPerSlot * kRegion == kTileBytes, "exchange regions");
        int8_t* region = (wu / kPerSlot == 0 ? slot_a(sa) : slot_b(sb)) + (wu % kPerSlot) * kRegion;
        const bool has_region = wu < 2 * kPerSlot;  // every wave that holds outputs
        const int c0 = sk_owner((int64_t)t * nk), c1 = sk_owner((int64_t)(t + 1) * nk - 1);
        for (int c = c0; c <= c1; ++c) {
            if (c == bid) continue;
            const __amdgpu_buffer_rsrc_t rs = slot_rsrc(c);
#pragma unroll
            for (int i0 = 0; i0 < 4; i0 += kRows) {
                if (has_region) {
#pragma unroll
                    for (int di = 0; di < kRows; ++di)
#pragma unroll
                        for (int j = 0; j < NJ; ++j)
                            if (block_live(i0 + di, j))
#pragma unroll
                                for (int q = 0; q < 4; ++q)
                                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                                        rs, (lds_ptr_t)(region + ((di * NJ + j) * 4 + q) * 1024), 16, (int)lane_off,
                                        (int)piece(i0 + di, j, q), 0, kCoherent);
                    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
                    for (int di = 0; di < kRows; ++di)
#pragma unroll
                        for (int j = 0; j < NJ; ++j)
                            if (block_live(i0 + di, j))
#pragma unroll
                                for (int q = 0; q < 4; ++q) {
                                    const v4i v = *(const v4i*)(region + ((di * NJ + j) * 4 + q) * 1024 + 16 * lane);
#pragma unroll
                                    for (int e = 0; e < 4; ++e) acc[i0 + di][j][4 * q + e] += v[e];
                                }
                    // this wave's reads are done before its region is loaded again
                    __builtin_amdgcn_s_waitcnt(0xC07F);
                }
            }
        }
        // every wave is done with the regions before the slots are written again (the
        // epilogue's factor table and staging)
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_s_barrier();
        return true;
    };

    // ---- prologue: global stages 0 and (of the long-lead operand) 1 in flight
    if constexpr (SK) {
        issue_a(0, k_0, 0);
        issue_b(0, k_0, 0);
        if (n_0 > 1) issue_b(1, k_0 + 1, 0);
        else issue_b(1, k_1, 1);
    } else {
        issue_a(0, 0, 0);
        issue_b(0, 0, 0);
        issue_b(1, nk > 1 ? 1 : 0, nk > 1 ? 0 : 1);
    }
    LLMINT8_WAIT_BARRIER(4);
    if constexpr (HALF && !ACC_OUT) {
        // rows 128..255 hold no valid row: the same loads and barriers as the other waves
        // (the stream-K exchange skips blocks without valid rows, and the epilogue needs only
        // this wave's entries of the factor tables)
        if (wu >= 4) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j) acc[i][j] = v16i{};
            int sa = 0, sb = 0;
            for (int ti = 0; ti < my_tiles; ++ti) {
                const int len = SK ? __builtin_amdgcn_readfirstlane(seg_n(ti)) : nk;
                for (int kt = 0; kt + 1 < len; ++kt) {
                    idle_stage(sa, sb, kt, ti, std::false_type{});
                    sa ^= 1;
                    sb = sb == 2 ? 0 : sb + 1;
                }
                idle_stage(sa, sb, len - 1, ti, std::true_type{});
                bool fin = true;
                if constexpr (SK) fin = sk_finish(ti, sa, sb);
                if (fin) {
                    float* rsc = (float*)slot_a(sa);
                    rsc[tid] = sc / 127.0f;
                    __builtin_amdgcn_s_waitcnt(0xC07F);
                    __builtin_amdgcn_s_barrier();
                }
                sa ^= 1;
                sb = sb == 2 ? 0 : sb + 1;
                if (ti + 1 < my_tiles) {
                    ra0 = ra1;
                    rb0 = rb1;
                    ra1 = ra2;
                    rb1 = rb2;
                    tile_rsrc(ti + 3, ra2, rb2);
                    __builtin_amdgcn_s_waitcnt(0xC07F);
                    __builtin_amdgcn_s_barrier();
                }
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            return;
        }
    }
    read_frags(0, 0, 0, fa[0], fb[0]);
    int sa = 0, sb = 0;
    for (int ti = 0; ti < my_tiles; ++ti) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j) acc[i][j] = v16i{};
        const int len = SK ? __builtin_amdgcn_readfirstlane(seg_n(ti)) : nk;
        for (int kt = 0; kt + 1 < len; ++kt) {
            stage(sa, sb, kt, ti, std::false_type{});
            sa ^= 1;
            sb = sb == 2 ? 0 : sb + 1;
        }
        stage(sa, sb, len - 1, ti, std::true_type{});
        if constexpr (SK) {
            if (sk_finish(ti, sa, sb)) epilogue(ti, sa, sb);
        } else {
            epilogue(ti, sa, sb);
        }
        sa ^= 1;
        sb = sb == 2 ? 0 : sb + 1;
        if (ti + 1 < my_tiles) {
            ra0 = ra1;
            rb0 = rb1;
            ra1 = ra2;
            rb1 = rb2;
            tile_rsrc(ti + 3, ra2, rb2);
            int lx = lane;
            asm volatile("" : "+v"(lx));
            lane_offsets(lx);
            // every wave is done with its staging area (the next stage's loads go there)
            __builtin_amdgcn_s_waitcnt(0xC07F);
            __builtin_amdgcn_s_barrier();
            read_frags(sa, sb, 0, fa[0], fb[0]);
        }
    }
    // no load into this workgroup's LDS may outlive it
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <int DT, bool ACC_OUT, bool HALF>
hipError_t launch_one(const Params& p, hipStream_t stream) {
    // persistent: one workgroup per compute unit (its LDS admits one), at most one per tile;
    // stream-K (one workgroup per compute unit) where the tiles leave the last round uneven
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    const int64_t T = (int64_t)p.tiles_m * p.tiles_n;
    const int64_t G = cus < kStreamKGrid ? cus : kStreamKGrid;
    if (p.sk_cnt != nullptr && p.sk_part != nullptr && G > 0 && T < 2 * G && T % G != 0) {
        // at most one workgroup per unit, so that every workgroup's range holds a stage (the
        // tile counts count the workgroups whose ranges meet the tile), and stream_k_per_tile
        // per tile; the workspace holds slots for stream_k_grid(M, K, N) >= g workgroups
        const int64_t g = stream_k_grid(p.M, p.K, p.N, G);
        gemm_kernel<DT, ACC_OUT, true, HALF><<<(unsigned)g, 64 * kWaves, 0, stream>>>(p);
        return hipGetLastError();
    }
    const int64_t wgs = T < cus ? T : (cus > 0 ? cus : 1);
    gemm_kernel<DT, ACC_OUT, false, HALF><<<(unsigned)wgs, 64 * kWaves, 0, stream>>>(p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream) {
    if (a.M == 0 || a.N == 0) return hipSuccess;
    if (a.K == 0) {
        // the empty sum: C = 0, F = 0, Y = +0 (the kernel assumes at least one K stage)
        const int64_t mn = a.M * a.N;
        if (a.Y) return launch_fill_zero((float*)a.Y, mn / 2, stream);  // N is a multiple of 8
        hipError_t e = launch_fill_zero((float*)a.C_acc, mn, stream);
        return e == hipSuccess ? launch_fill_zero(a.F_acc, mn, stream) : e;
    }
    Params p;
    p.Xq = a.Xq;
    p.xq_pitch = a.xq_pitch;
    p.Wq = a.Wq;
    p.M = a.M;
    p.N = a.N;
    p.K = a.K;
    p.s_x = a.s_x;
    p.s_w = a.s_w;
    p.XO = (const uint16_t*)a.XO;
    p.WO = (const uint16_t*)a.WO;
    p.xo_pitch = a.xo_pitch;
    p.wo_pitch = a.wo_pitch;
    p.f_scaled = a.f_scaled ? 1 : 0;
    p.n_out = a.n_out;
    p.Y = (uint16_t*)a.Y;
    p.C_acc = a.C_acc;
    p.F_acc = a.F_acc;
    p.tiles_m = (int)ceil_div(a.M, BM);
    p.tiles_n = (int)ceil_div(a.N, BN);
    p.sk_cnt = a.sk_cnt;
    p.sk_part = a.sk_part;
    const bool acc_out = a.Y == nullptr, half = a.M <= BM / 2;
    if (acc_out) return a.dt == F16 ? launch_one<F16, true, false>(p, stream) : launch_one<BF16, true, false>(p, stream);
    if (a.dt == F16) return half ? launch_one<F16, false, true>(p, stream) : launch_one<F16, false, false>(p, stream);
    return half ? launch_one<BF16, false, true>(p, stream) : launch_one<BF16, false, false>(p, stream);
}

}  // namespace llmint8
