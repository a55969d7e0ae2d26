// Group-wise scales along K: one absmax scale per group of G consecutive input features,
// for every row of X and every column of W (the finer granularity the "nuQmm" report page
// discusses for weight quantization; here for both operands, without the outlier
// decomposition).  G is a power of two, G >= 128 and G divides K; ng = K / G.
//   s_x[i*ng + g], Xq[i,k]: the vector-wise code of each row group;
//   s_w[n*ng + g], Wq[n,k]: the same for each column group of W;
//   C_g = Xq_g Wq_g^T (exact int32), and per output element
//   acc = 0; for g ascending: acc = RN32(acc + RN32(RN32((float)C_g * r_ig) * c_ng)),
//   r_ig = RN32(s_x/127), c_ng = RN32(s_w/127);  Y = RN_T(acc).
//
// Product kernel: the tiled int8 MFMA kernel's scheme (K stages of 128 bytes loaded
// straight into LDS, counted waits, XOR chunk swizzle, XCD-contiguous tile order) with a
// 256 x 128 tile over 8 waves (4 x 2, two per SIMD), each 64 x 64: 64 int32 partials and
// 64 fp32 sums per lane in its 256 registers.  Both operands are loaded two stages ahead
// (3 + 3 slots).  A group's first products start from zero; after its last stage every
// wave folds its int32 partials into the fp32 sums -- while it does, the other wave on its
// SIMD keeps the matrix unit busy.  The group's factors come through LDS: r (precomputed by the X pass, group-major)
// and s_w for the tile's rows and columns, loaded straight into LDS at the group's first
// stage, before the stage's operand loads, so the counted wait and barrier that cover
// stage kt+1 cover them too; two slots alternate between groups.
// Persistent: one workgroup per compute unit works through its XCD's run of tiles; the K
// stages run back to back across tile boundaries (a tile's last stages already load the
// next tile's first operands), and a tile's epilogue stages Y through the slots of the
// stage it consumed last while those loads are in flight.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace llmint8 {

namespace {

constexpr int NJ = 2;                           // 32-column MFMA tiles per wave along N
constexpr int MI = 2;                           // 32-row MFMA tiles per wave along M
constexpr int kWaves = 8;                       // 4 (M) x 2 (N), two per SIMD, 64 x 64 each
constexpr int BM = 4 * 32 * MI, BN = 2 * 32 * NJ;  // 256 x 128
constexpr int BK = 128;
constexpr int kTileBytesA = BM * BK;            // 32 KB
constexpr int kTileBytesB = BN * BK;            // 16 KB
constexpr int kChunks = BK / 16;
constexpr int kRowsPerLoad = 64 / kChunks;      // 8
constexpr int kLoadsA = BM / kRowsPerLoad / kWaves;  // 4 per wave and stage
constexpr int kLoadsB = BN / kRowsPerLoad / kWaves;  // 2 per wave and stage
// Both operands are loaded two stages ahead (three slots each: 144 KB).
constexpr int kSlotsA = 3, kSlotsB = 3;
constexpr int kOperandBytes = kSlotsA * kTileBytesA + kSlotsB * kTileBytesB;
constexpr int kScaleBytes = 2 * (BM + BN) * 4;                                // two slots of r and s_w
constexpr int kSubSteps = BK / 32;
constexpr int kGroupM = 8;
constexpr int kXcds = 8;
constexpr int kYPitch = 32 * NJ + 8;             // epilogue staging row, 16-bit elements
constexpr int kYHalfBytes = 32 * kYPitch * 2;      // one 32-row half of a wave's outputs
static_assert(kOperandBytes + kScaleBytes <= 160 * 1024, "LDS");
static_assert(6 * kYHalfBytes <= kTileBytesA && 2 * kYHalfBytes <= kTileBytesB, "epilogue LDS");
static_assert(kLoadsA + kLoadsB == 6, "the barrier's wait leaves the 6 loads of stage kt+2 in flight");

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Every lambda of the product kernel is inlined: one left out of line would take the
// accumulator arrays it captures by reference into private (scratch) memory.
#define LLMINT8_INLINE __attribute__((always_inline))

// Operand loads: a raw buffer resource over the tile's rows (dword data format), 32-bit
// offsets, the stage's K position in the scalar offset; 16 bytes per lane into LDS.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rs, uint32_t voffset, int soffset, int8_t* lds) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)lds, 16, (int)voffset, soffset, 0, 0);
}

__host__ __device__ constexpr int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

#define LLMINT8_GROUP_WAIT_BARRIER(N)                                              \
    do {                                                                           \
        __builtin_amdgcn_s_waitcnt(0xC07F);                                        \
        asm volatile("s_waitcnt vmcnt(" #N ")\n\ts_barrier" ::: "memory");         \
    } while (0)

struct GroupParams {
    const int8_t* Xq;   // M x K (pitch K)
    const float* rg;    // ng x M: r = RN32(s_x / 127), group-major
    const int8_t* Wq;   // N x K
    const float* s_w;   // N x ng
    int64_t M, N, K, ng;
    int gs;             // K stages per group (G / 128)
    uint16_t* Y;
    int tiles_m, tiles_n;
};

template <int DT>
__global__ __launch_bounds__(64 * kWaves) void gemm_group_kernel(GroupParams p) {
    __shared__ __attribute__((aligned(1024))) int8_t smem[kOperandBytes + kScaleBytes];
    float* rbuf = (float*)(smem + kOperandBytes);  // [2][BM]
    float* cbuf = rbuf + 2 * BM;                   // [2][BN]: s_w of the tile's columns
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w >> 1, wn = w & 1;

    // ---- tiles of this workgroup: the XCD-contiguous run of tiles (grouped order) of the
    // XCD the dispatcher places it on (ids congruent mod 8), strided by the number of
    // workgroups on that XCD
    const int T = p.tiles_m * p.tiles_n;
    const int bid = blockIdx.x, nwg = gridDim.x;
    const int xcd = bid % kXcds, local = bid / kXcds;
    const int per = T / kXcds, rem = T % kXcds;
    const int x_start = xcd * per + (xcd < rem ? xcd : rem), x_cnt = per + (xcd < rem ? 1 : 0);
    const int on_xcd = (nwg - xcd + kXcds - 1) / kXcds;
    const int my_tiles = local < x_cnt ? (x_cnt - local + on_xcd - 1) / on_xcd : 0;
    if (my_tiles == 0) return;  // the same for every wave of the workgroup
    auto tile_origin = [&](int i, int64_t& m0, int64_t& n0) LLMINT8_INLINE {
        const int t = x_start + local + i * on_xcd;
        const int in_group = kGroupM * p.tiles_n;
        const int first_m = (t / in_group) * kGroupM;
        const int gm = p.tiles_m - first_m < kGroupM ? p.tiles_m - first_m : kGroupM;
        m0 = (int64_t)(first_m + (t % in_group) % gm) * BM;
        n0 = (int64_t)((t % in_group) / gm) * BN;
    };

    // ---- per-lane offsets, relative to a tile's first row: operand rows (one 128-byte
    // line each, swizzled chunks) and the factor entries; rows past M or N lie past the
    // resources and read zero
    const int wu = __builtin_amdgcn_readfirstlane(w);
    uint32_t a_off[kLoadsA], b_off[kLoadsB];
#pragma unroll
    for (int j = 0; j < kLoadsA; ++j) {
        const int r = kRowsPerLoad * (kLoadsA * wu + j) + lane / kChunks;
        a_off[j] = (uint32_t)(r * p.K + (((lane % kChunks) ^ swz(r)) << 4));
    }
#pragma unroll
    for (int j = 0; j < kLoadsB; ++j) {
        const int r = kRowsPerLoad * (kLoadsB * wu + j) + lane / kChunks;
        b_off[j] = (uint32_t)(r * p.K + (((lane % kChunks) ^ swz(r)) << 4));
    }
    const int nk = (int)(p.K / BK);  // K is a multiple of G >= 128
    // Loads run two stages ahead, across tile boundaries: the resources of this tile and
    // the next two are held; past the workgroup's last tile they are empty (every stage
    // issues its loads, which then land zeros in slots no stage reads).
    auto tile_rsrc = [&](int i, __amdgpu_buffer_rsrc_t& ra, __amdgpu_buffer_rsrc_t& rb) LLMINT8_INLINE {
        int64_t m0 = 0, n0 = 0, rows_a = 0, rows_b = 0;
        if (i < my_tiles) {
            tile_origin(i, m0, n0);
            rows_a = p.M - m0 < BM ? p.M - m0 : BM;
            rows_b = p.N - n0 < BN ? p.N - n0 : BN;
        }
        ra = buffer_rsrc(p.Xq + m0 * p.K, rows_a * p.K);
        rb = buffer_rsrc(p.Wq + n0 * p.K, rows_b * p.K);
    };
    __amdgpu_buffer_rsrc_t ra0, rb0, ra1, rb1, ra2, rb2;
    tile_rsrc(0, ra0, rb0);
    tile_rsrc(1, ra1, rb1);
    tile_rsrc(2, ra2, rb2);

    // global stage s sits in slot s % 3 of each operand; `d` = tiles ahead of the current one
    auto slot_a = [&](int ss) LLMINT8_INLINE { return smem + ss * kTileBytesA; };
    auto slot_b = [&](int ss) LLMINT8_INLINE { return smem + kSlotsA * kTileBytesA + ss * kTileBytesB; };
    auto issue_ab = [&](int ss, int kt, int d) LLMINT8_INLINE {
        const __amdgpu_buffer_rsrc_t rs_a = d == 0 ? ra0 : (d == 1 ? ra1 : ra2);
        const __amdgpu_buffer_rsrc_t rs_b = d == 0 ? rb0 : (d == 1 ? rb1 : rb2);
        int8_t* As = slot_a(ss);
        int8_t* Bs = slot_b(ss);
#pragma unroll
        for (int j = 0; j < kLoadsA; ++j) load_lds16(rs_a, a_off[j], kt * BK, As + (kLoadsA * wu + j) * 1024);
#pragma unroll
        for (int j = 0; j < kLoadsB; ++j) load_lds16(rs_b, b_off[j], kt * BK, Bs + (kLoadsB * wu + j) * 1024);
    };
    // the factors of group g of the current tile, one 64-entry load per wave: waves 0..3 the
    // r of the tile's 256 rows, waves 4 and 5 the s_w of its 128 columns, waves 6 and 7 the
    // same columns again (same values to the same place, so that every wave issues the same
    // loads)
    const int cw = wu & 1;
    const uint32_t r_off = (uint32_t)((64 * (wu & 3) + lane) * 4);
    const uint32_t c_off = (uint32_t)((64 * cw + lane) * p.ng * 4);
    int64_t cm0 = 0, cn0 = 0;  // the current tile's origin
    tile_origin(0, cm0, cn0);
    auto issue_scales = [&](int g) LLMINT8_INLINE {
        const int64_t rows_a = p.M - cm0 < BM ? p.M - cm0 : BM, rows_b = p.N - cn0 < BN ? p.N - cn0 : BN;
        const __amdgpu_buffer_rsrc_t rs = wu < 4 ? buffer_rsrc(p.rg + (int64_t)g * p.M + cm0, rows_a * 4)
                                                 : buffer_rsrc(p.s_w + cn0 * p.ng + g, rows_b * p.ng * 4);
        float* dst = wu < 4 ? rbuf + (g & 1) * BM + 64 * wu : cbuf + (g & 1) * BN + 64 * cw;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)dst, 4, (int)(wu < 4 ? r_off : c_off), 0, 0, 0);
    };

    const int rl = lane & 31, h = lane >> 5;
    int rd[kSubSteps];
#pragma unroll
    for (int u = 0; u < kSubSteps; ++u) rd[u] = rl * BK + (((2 * u + h) ^ swz(rl)) << 4);
    auto read_frags = [&](int ss, int u, v4i (&fa)[MI], v4i (&fb)[NJ]) LLMINT8_INLINE {
        const int8_t* As = slot_a(ss) + wm * (32 * MI) * BK + rd[u];
        const int8_t* Bs = slot_b(ss) + wn * (32 * NJ) * BK + rd[u];
        fa[0] = *(const v4i*)As;
#pragma unroll
        for (int j = 0; j < NJ; ++j) fb[j] = *(const v4i*)(Bs + j * 32 * BK);
#pragma unroll
        for (int i = 1; i < MI; ++i) fa[i] = *(const v4i*)(As + i * 32 * BK);
    };

    v16i acc[MI][NJ];
    v16f accf[MI][NJ];
    // ZERO: the group's first products, which start from 0 instead of the previous group's
    // partial (so the partials are never cleared)
    auto mfma_rows = [&](const v4i (&fa)[MI], const v4i (&fb)[NJ], int i0, int i1, auto zero_tag) LLMINT8_INLINE {
        constexpr bool ZERO = decltype(zero_tag)::value;
#pragma unroll
        for (int i = i0; i < i1; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[i], fb[j], ZERO ? v16i{} : acc[i][j], 0, 0, 0);
    };
    // fold group g into the fp32 sums (lane: column 32j + lane%32 of the wave's 64, rows
    // 8*(e/4) + 4*(lane/32) + e%4 of each 32-row slice)
    auto fold = [&](int g) LLMINT8_INLINE {
        const float* rb = rbuf + (g & 1) * BM + wm * (32 * MI);
        const float* cb = cbuf + (g & 1) * BN + wn * 64;
        float c[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) c[j] = cb[32 * j + rl] / 127.0f;
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            float r[16];
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const v4f t4 = *(const v4f*)(rb + 32 * i + 8 * a + 4 * h);
#pragma unroll
                for (int b = 0; b < 4; ++b) r[4 * a + b] = t4[b];
            }
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    accf[i][j][e] = __fadd_rn(accf[i][j][e], __fmul_rn(__fmul_rn((float)acc[i][j][e], r[e]), c[j]));
            // one 32-row slice at a time: hoisting every partial's read would need 128 more
            // registers than the sums and the next operands leave
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // One K stage (global stage in slot ss, stage kt of its tile): sub-steps 0..2 run their 8
    // MFMAs under the next sub-step's 6 LDS reads and, in sub-step 0 of a group's first
    // stage, the loads of the group's factors, in sub-step 1 the global loads two stages
    // ahead (both operands, into the slots the previous stage freed); sub-step 3 runs 2
    // MFMAs, waits for the next stage and meets the other waves at the barrier, then reads
    // the next stage's first operands under its other 6.  FIRST: the group's first stage.
    v4i fa[2][MI], fb[2][NJ];
    auto stage = [&](int ss, int kt, int g, auto first_tag) LLMINT8_INLINE {
        constexpr bool FIRST = decltype(first_tag)::value;
        // (readfirstlane: the compiler then knows this, and so the resources, are uniform)
        const int d = __builtin_amdgcn_readfirstlane(kt + 2 < nk ? 0 : (kt + 2 < 2 * nk ? 1 : 2));
        const int k2 = kt + 2 - d * nk;
        const int s1 = ss == 2 ? 0 : ss + 1, s2 = ss == 0 ? 2 : ss - 1;
#pragma unroll
        for (int u = 0; u < kSubSteps - 1; ++u) {
            const int cur = u & 1, nxt = cur ^ 1;
            __builtin_amdgcn_s_waitcnt(0xC07F);
            if (u == 0 && FIRST) issue_scales(g);
            if (u == 1) issue_ab(s2, k2, d);
            read_frags(ss, u + 1, fa[nxt], fb[nxt]);
            if (u == 0) mfma_rows(fa[cur], fb[cur], 0, MI, std::integral_constant<bool, FIRST>{});
            else mfma_rows(fa[cur], fb[cur], 0, MI, std::false_type{});
            if (u == 1) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (q < 2) __builtin_amdgcn_sched_group_barrier(0x010, 2, 0);
                    else __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                }
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        mfma_rows(fa[1], fb[1], 0, 1, std::false_type{});
        __builtin_amdgcn_sched_barrier(0);
        LLMINT8_GROUP_WAIT_BARRIER(6);  // the loads two stages ahead may stay in flight
        read_frags(s1, 0, fa[0], fb[0]);
        mfma_rows(fa[1], fb[1], 1, MI, std::false_type{});
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_barrier(0);
    };

    // ---- epilogue of the current tile: Y = RN_T(sums), one 32-row half per wave at a time,
    // staged in the A and B slots of the stage just consumed (A: waves 0-5, B: waves 6, 7),
    // written as 16-byte row segments
    auto epilogue = [&](int ss) LLMINT8_INLINE {
        uint16_t* ys = (uint16_t*)(w < 6 ? slot_a(ss) + w * kYHalfBytes : slot_b(ss) + (w - 6) * kYHalfBytes);
        const int64_t wm0 = cm0 + wm * (32 * MI), wn0 = cn0 + wn * (32 * NJ);
        constexpr int kLanesPerRow = 32 * NJ / 8;  // 16-byte segments per staged row
        constexpr int kRowsPerIter = 64 / kLanesPerRow;
#pragma unroll
        for (int i = 0; i < MI; ++i) {
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    ys[(8 * (e >> 2) + 4 * h + (e & 3)) * kYPitch + 32 * j + rl] = from_f32<DT>(accf[i][j][e]);
#pragma unroll
            for (int it = 0; it < 32 / kRowsPerIter; ++it) {
                const int row = it * kRowsPerIter + lane / kLanesPerRow, ch = lane % kLanesPerRow;
                const u32x4 v = *(const u32x4*)(ys + row * kYPitch + ch * 8);
                const int64_t m = wm0 + 32 * i + row, n = wn0 + ch * 8;
                if (m < p.M && n < p.N) *(u32x4*)(p.Y + m * p.N + n) = v;
            }
        }
    };

    // prologue: global stages 0 and 1 in flight; wait for stage 0
    issue_ab(0, 0, 0);
    issue_ab(1, nk > 1 ? 1 : 0, nk > 1 ? 0 : 1);
    LLMINT8_GROUP_WAIT_BARRIER(6);
    read_frags(0, 0, fa[0], fb[0]);
    int ss = 0;
    for (int ti = 0; ti < my_tiles; ++ti) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j) accf[i][j] = v16f{};
        int kt = 0;
        for (int g = 0; g < (int)p.ng; ++g) {
            stage(ss, kt++, g, std::true_type{});
            ss = ss == 2 ? 0 : ss + 1;
            for (int s = 1; s < p.gs; ++s) {
                stage(ss, kt++, g, std::false_type{});
                ss = ss == 2 ? 0 : ss + 1;
            }
            fold(g);
        }
        // the stage just consumed sits in the slot before ss; no wave reads it any more
        epilogue(ss == 0 ? 2 : ss - 1);
        if (ti + 1 < my_tiles) {
            ra0 = ra1;
            rb0 = rb1;
            ra1 = ra2;
            rb1 = rb2;
            tile_rsrc(ti + 3, ra2, rb2);
            tile_origin(ti + 1, cm0, cn0);
            // every wave is done with its staging area (the next stage's loads go there)
            __builtin_amdgcn_s_waitcnt(0xC07F);
            __builtin_amdgcn_s_barrier();
        }
    }
    // no load into this workgroup's LDS may outlive it
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// ---- X pass: the group-wise codes of X.  Row groups never cross rows (G divides K), so X
// is a flat run of M * ng groups of G elements: SEG lanes take one group (SEG = 64, or 16 /
// 32 for G = 128 / 256), each lane NV 16-byte chunks of 8 elements, one wave access 1 KB.
// Xqb (nullable; used for G = 256 to 1024): the codes again, in the small-batch kernel's blocks
// (K is a multiple of G, hence of 64: no padding).
template <int DT, int NV, int SEG>
__global__ __launch_bounds__(256) void group_rows_kernel(const uint16_t* __restrict__ X, int64_t M, int64_t K,
                                                         int64_t G, int8_t* __restrict__ Xq, float* __restrict__ s_x,
                                                         float* __restrict__ rg, int8_t* __restrict__ Xqb) {
    constexpr int BPW = 64 / SEG;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int sub = lane / SEG, sl = lane % SEG;
    const int64_t ng = K / G, nblocks = M * ng;
    const int64_t nwaves = (int64_t)gridDim.x * 4;
    for (int64_t b0 = ((int64_t)blockIdx.x * 4 + w) * BPW; b0 < nblocks; b0 += nwaves * BPW) {
        const int64_t b = b0 + sub;
        const bool in = b < nblocks;
        const int64_t lo = (in ? b : 0) * G;
        u32x4 v[NV];
#pragma unroll
        for (int j = 0; j < NV; ++j) v[j] = in ? *(const u32x4*)(X + lo + 8 * ((int64_t)j * SEG + sl)) : u32x4{0u, 0u, 0u, 0u};
        uint32_t m = 0;
#pragma unroll
        for (int j = 0; j < NV; ++j)
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint32_t a = v[j][d] & 0x7fff7fffu;  // magnitudes: unsigned order = |x| order
                const uint32_t lo16 = a & 0xffffu, hi16 = a >> 16;
                m = m > lo16 ? m : lo16;
                m = m > hi16 ? m : hi16;
            }
#pragma unroll
        for (int off = SEG / 2; off > 0; off >>= 1) {
            const uint32_t o = (uint32_t)__shfl_xor((int)m, off, kWave);
            m = m > o ? m : o;
        }
        const float s = to_f32<DT>((uint16_t)m);
        const float inv = inv_scale(s);
        int8_t* qb = nullptr;  // groups of at most 1024 (NV <= 2): more would cost occupancy here
        if constexpr (NV <= 2) qb = Xqb && in ? Xqb + xqb_offset(b / ng, (b % ng) * G + 8 * sl, K / 64) : nullptr;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            uint32_t t[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                float f = __fmul_rn(to_f32<DT>((uint16_t)(v[j][k >> 1] >> (16 * (k & 1)))), inv);
                f = fminf(fmaxf(f, -127.0f), 127.0f);
                t[k] = __builtin_bit_cast(uint32_t, __fadd_rn(f, 12582912.0f));  // rne into the low byte
            }
            u32x2 q;
            q[0] = __builtin_amdgcn_perm(t[1], t[0], 0x0c0c0400u) | __builtin_amdgcn_perm(t[3], t[2], 0x04000c0cu);
            q[1] = __builtin_amdgcn_perm(t[5], t[4], 0x0c0c0400u) | __builtin_amdgcn_perm(t[7], t[6], 0x04000c0cu);
            if (in) {
                *(u32x2*)(Xq + lo + 8 * ((int64_t)j * SEG + sl)) = q;
                // chunk j lies 8 SEG columns (8 SEG / 64 blocks of 1 KB) past chunk 0
                if (qb) *(u32x2*)(qb + (int64_t)j * SEG * 128) = q;
            }
        }
        if (sl == 0 && in) {
            const int64_t i = b / ng, g = b % ng;
            s_x[b] = s;                    // row-major: i * ng + g
            rg[g * M + i] = s / 127.0f;    // group-major dequantization factor
        }
    }
}

// ---- weight scales: s_w[n*ng + g] = max |W[k,n]| over group g; one workgroup per (512
// columns, group), its four waves split the group's rows, no atomics.
template <int DT>
__global__ __launch_bounds__(256) void group_colmax_kernel(const uint16_t* __restrict__ W, int64_t K, int64_t N,
                                                           int64_t G, float* __restrict__ s_w) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t n8 = ((int64_t)blockIdx.x * 64 + lane) * 8;
    const int64_t g = blockIdx.y, ng = K / G;
    float m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (n8 < N) {
        for (int64_t k = g * G + w; k < (g + 1) * G; k += 4) {
            const u32x4 v = *(const u32x4*)(W + k * N + n8);
#pragma unroll
            for (int j = 0; j < 8; ++j)
                m[j] = fmaxf(m[j], __builtin_fabsf(to_f32<DT>((uint16_t)(v[j >> 1] >> (16 * (j & 1))))));
        }
    }
    __shared__ float sm[4][64][9];
#pragma unroll
    for (int j = 0; j < 8; ++j) sm[w][lane][j] = m[j];
    __syncthreads();
    if (w == 0 && n8 < N) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            s_w[(n8 + j) * ng + g] = fmaxf(fmaxf(sm[0][lane][j], sm[1][lane][j]), fmaxf(sm[2][lane][j], sm[3][lane][j]));
    }
}

template <int DT, int NV, int SEG>
hipError_t group_rows_launch(const void* X, int64_t M, int64_t K, int64_t G, int8_t* Xq, float* s_x, float* rg,
                             int8_t* Xqb, hipStream_t stream) {
    const int64_t nblocks = M * (K / G);
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus = 256;
    const int64_t need = ceil_div(nblocks, 4 * (64 / SEG));
    const unsigned grid = (unsigned)(need < (int64_t)cus * 8 ? need : (int64_t)cus * 8);
    group_rows_kernel<DT, NV, SEG><<<grid, 256, 0, stream>>>((const uint16_t*)X, M, K, G, Xq, s_x, rg, Xqb);
    return hipGetLastError();
}

template <int DT>
hipError_t group_rows_dispatch(const void* X, int64_t M, int64_t K, int64_t G, int8_t* Xq, float* s_x, float* rg,
                               int8_t* Xqb, hipStream_t stream) {
    switch (G) {
        case 128: return group_rows_launch<DT, 1, 16>(X, M, K, G, Xq, s_x, rg, Xqb, stream);
        case 256: return group_rows_launch<DT, 1, 32>(X, M, K, G, Xq, s_x, rg, Xqb, stream);
        case 512: return group_rows_launch<DT, 1, 64>(X, M, K, G, Xq, s_x, rg, Xqb, stream);
        case 1024: return group_rows_launch<DT, 2, 64>(X, M, K, G, Xq, s_x, rg, Xqb, stream);
        case 2048: return group_rows_launch<DT, 4, 64>(X, M, K, G, Xq, s_x, rg, Xqb, stream);
        default: return group_rows_launch<DT, 8, 64>(X, M, K, G, Xq, s_x, rg, Xqb, stream);  // 4096
    }
}

}  // namespace

bool group_size_ok(int64_t G, int64_t K) { return G >= 128 && G <= 4096 && (G & (G - 1)) == 0 && K % G == 0; }

hipError_t launch_group_xpass(int dt, const void* X, int64_t M, int64_t K, int64_t G, int8_t* Xq, float* s_x,
                              float* rg, int8_t* Xqb, hipStream_t stream) {
    if (M == 0 || K == 0) return hipSuccess;
    return dt == F16 ? group_rows_dispatch<F16>(X, M, K, G, Xq, s_x, rg, Xqb, stream)
                     : group_rows_dispatch<BF16>(X, M, K, G, Xq, s_x, rg, Xqb, stream);
}

hipError_t launch_group_colmax(int dt, const void* W, int64_t K, int64_t N, int64_t G, float* s_w,
                               hipStream_t stream) {
    if (N == 0 || K == 0) return hipSuccess;
    dim3 g((unsigned)ceil_div(N, 512), (unsigned)(K / G));
    if (dt == F16) group_colmax_kernel<F16><<<g, 256, 0, stream>>>((const uint16_t*)W, K, N, G, s_w);
    else group_colmax_kernel<BF16><<<g, 256, 0, stream>>>((const uint16_t*)W, K, N, G, s_w);
    return hipGetLastError();
}

hipError_t launch_gemm_group(int dt, const int8_t* Xq, const float* rg, const int8_t* Wq, const float* s_w, int64_t M,
                             int64_t N, int64_t K, int64_t G, void* Y, hipStream_t stream) {
    if (M == 0 || N == 0) return hipSuccess;
    GroupParams p;
    p.Xq = Xq;
    p.rg = rg;
    p.Wq = Wq;
    p.s_w = s_w;
    p.M = M;
    p.N = N;
    p.K = K;
    p.ng = K / G;
    p.gs = (int)(G / BK);
    p.Y = (uint16_t*)Y;
    p.tiles_m = (int)ceil_div(M, BM);
    p.tiles_n = (int)ceil_div(N, BN);
    // persistent: one workgroup per compute unit (its LDS admits one), at most one per tile
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    const int64_t T = (int64_t)p.tiles_m * p.tiles_n;
    const unsigned grid = (unsigned)(T < cus ? T : (cus > 0 ? cus : 1));
    if (dt == F16) gemm_group_kernel<F16><<<grid, 64 * kWaves, 0, stream>>>(p);
    else gemm_group_kernel<BF16><<<grid, 64 * kWaves, 0, stream>>>(p);
    return hipGetLastError();
}

}  // namespace llmint8
