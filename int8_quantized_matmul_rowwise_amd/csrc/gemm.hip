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
constexpr int kGroupM = 8;
// epilogue staging (reuses the operand slots): the tile's row and column factors, then per
// wave its 128 x 64 outputs, rows padded to 144 bytes (16-byte aligned)
constexpr int kScaleBytes = 2 * 256 * 4;
constexpr int kYPitch = 72;  // 16-bit elements
constexpr int kYStageBytes = 128 * kYPitch * 2;                               // row tiles per group of the tile order
constexpr int kXcds = 8;
static_assert(kSlotsA * kTileBytes + kSlotsB * kSlotBytesB <= 160 * 1024, "LDS");
static_assert(kLoadsA == 4 && kLoadsB == 4, "the waits below count 4 loads per operand and wave");
static_assert(kScaleBytes + kWaves * kYStageBytes <= kSlotsA * kTileBytes + kSlotsB * kSlotBytesB, "epilogue LDS");
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
};

template <int DT>
__device__ __forceinline__ v16f mfma16(const u32x4& a, const u32x4& b, const v16f& c) {
    if constexpr (DT == F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, a), __builtin_bit_cast(v8h, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
}

template <int DT, bool ACC_OUT>
__global__ __launch_bounds__(64 * kWaves) void gemm_kernel(Params p) {
    __shared__ __attribute__((aligned(1024))) int8_t smem[kSlotsA * kTileBytes + kSlotsB * kSlotBytesB];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w >> 2, wn = w & 3;

    // ---- tile of this workgroup (XCD-contiguous runs, grouped order)
    const int T = p.tiles_m * p.tiles_n;
    const int bid = blockIdx.x;
    const int xcd = bid % kXcds, local = bid / kXcds;
    const int per = T / kXcds, rem = T % kXcds;
    const int t = xcd * per + (xcd < rem ? xcd : rem) + local;
    const int in_group = kGroupM * p.tiles_n;
    const int first_m = (t / in_group) * kGroupM;
    const int gm = p.tiles_m - first_m < kGroupM ? p.tiles_m - first_m : kGroupM;
    const int tm = first_m + (t % in_group) % gm;
    const int tn = (t % in_group) / gm;
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

    // ---- loader: wave w fills LDS slots [1024*(4w+j), +1024) of each operand, j = 0..3:
    // row r = 8*(4w + j) + lane/8 (one 128-byte line per row), physical chunk lane%8,
    // logical chunk (lane%8) ^ swz(r).
    const int wu = __builtin_amdgcn_readfirstlane(w);
    uint32_t a_off[kLoadsA], b_off[kLoadsB];
#pragma unroll
    for (int j = 0; j < kLoadsA; ++j) {
        const int r = kRowsPerLoad * (kLoadsA * wu + j) + lane / kChunks;
        const int c = (lane % kChunks) ^ swz(r);
        const int64_t m = m0 + r < p.M ? m0 + r : p.M - 1;
        a_off[j] = (uint32_t)((m - m0) * p.xq_pitch + c * 16);
    }
#pragma unroll
    for (int j = 0; j < kLoadsB; ++j) {
        const int r = kRowsPerLoad * (kLoadsB * wu + j) + lane / kChunks;
        const int c = (lane % kChunks) ^ swz(r);
        const int64_t n = n0 + r < p.N ? n0 + r : p.N - 1;
        b_off[j] = (uint32_t)((n - n0) * p.K + c * 16);
    }
    const int8_t* a_tile = p.Xq + m0 * p.xq_pitch;
    const int8_t* b_tile = p.Wq + n0 * p.K;
    const int nk = (int)ceil_div(p.K, BK);
    // The resources span the tile's rows (at most 256 of them: offsets fit 32 bits for any
    // K the library accepts).  In a partial last stage the chunks past K of a B row read the
    // next row's first bytes, or nothing (zero) past the last row: their A side is the zero
    // padding of Xq, so they add exact zeros.
    const int64_t rows_a = p.M - m0 < BM ? p.M - m0 : BM, rows_b = p.N - n0 < BN ? p.N - n0 : BN;
    const __amdgpu_buffer_rsrc_t rsa = buffer_rsrc(a_tile, rows_a * p.xq_pitch);
    const __amdgpu_buffer_rsrc_t rsb = buffer_rsrc(b_tile, rows_b * p.K);

    auto slot_a = [&](int kt) { return smem + (kt % kSlotsA) * kTileBytes; };
    auto slot_b = [&](int kt) { return smem + kSlotsA * kTileBytes + (kt % kSlotsB) * kSlotBytesB; };
    auto issue_a = [&](int kt) {
        int8_t* As = slot_a(kt);
        const int kb = kt * BK;
#pragma unroll
        for (int j = 0; j < kLoadsA; ++j) load_lds16(rsa, a_off[j], kb, As + (kLoadsA * wu + j) * 1024);
    };
    auto issue_b = [&](int kt) {
        int8_t* Bs = slot_b(kt);
        const int kb = kt * BK;
#pragma unroll
        for (int j = 0; j < kLoadsB; ++j) load_lds16(rsb, b_off[j], kb, Bs + (kLoadsB * wu + j) * 1024);
    };

    // ---- MFMA operand reads (32x32x32: lane holds row lane%32, 16 k at 16*(lane/32)):
    // fragment i of sub-step u reads row 32*i + lane%32 of the wave's 128-row panel,
    // logical chunk 2u + lane/32.  Read in the order the MFMAs consume them.
    const int rl = lane & 31, h = lane >> 5;
    int rd[kSubSteps];
#pragma unroll
    for (int u = 0; u < kSubSteps; ++u) rd[u] = rl * BK + (((2 * u + h) ^ swz(rl)) << 4);
    auto read_frags = [&](int kt, int u, v4i (&fa)[4], v4i (&fb)[NJ]) {
        const int8_t* As = slot_a(kt) + wm * 128 * BK + rd[u];
        const int8_t* Bs = slot_b(kt) + wn * (32 * NJ) * BK + rd[u];
        fa[0] = *(const v4i*)As;
#pragma unroll
        for (int j = 0; j < NJ; ++j) fb[j] = *(const v4i*)(Bs + j * 32 * BK);
#pragma unroll
        for (int i = 1; i < 4; ++i) fa[i] = *(const v4i*)(As + i * 32 * BK);
    };

    v16i acc[4][NJ];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = v16i{};

    auto mfma_rows = [&](const v4i (&fa)[4], const v4i (&fb)[NJ], int i0, int i1) {
#pragma unroll
        for (int i = i0; i < i1; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
    };

    // One K stage.  Sub-steps 0..2 run their 8 MFMAs while the 6 LDS reads of the next
    // sub-step (and, in 0 and 1, the global loads of stage kt+1 of the short-lead operand
    // and stage kt+2 of the long-lead one, into the slots stage kt-1 freed) are
    // interleaved, front-loaded so they have most of the sub-step to land.  Sub-step 3 runs
    // 2 MFMAs, waits for stage kt+1 and meets the other waves at the barrier, then reads
    // stage kt+1's first operands under its other 6.  Each sub-step is fenced
    // (sched_barrier) so that the interleave stays inside it.
    // STEADY: stage kt+2 exists (every stage but the last two).
    v4i fa[2][4], fb[2][NJ];  // operand sets of the current / next sub-step
    auto stage = [&](int kt, auto steady_tag) {
        constexpr bool STEADY = decltype(steady_tag)::value;
        const bool next = STEADY || kt + 1 < nk;
#pragma unroll
        for (int u = 0; u < kSubSteps - 1; ++u) {
            const int cur = u & 1, nxt = cur ^ 1;
            const bool loads = STEADY && u < 2;
            // this sub-step's operands were read a sub-step ago: a free wait that keeps the
            // compiler's own waits (it counts the direct-to-LDS loads as LDS traffic) out
            __builtin_amdgcn_s_waitcnt(0xC07F);
            if (u == 0 && next) {
                if (kLeadA) issue_b(kt + 1);
                else issue_a(kt + 1);
            }
            if (u == 1 && STEADY) {
                if (kLeadA) issue_a(kt + 2);
                else issue_b(kt + 2);
            }
            read_frags(kt, u + 1, fa[nxt], fb[nxt]);
            mfma_rows(fa[cur], fb[cur], 0, 4);
            if (loads) {
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
        if constexpr (STEADY) LLMINT8_WAIT_BARRIER(4);  // the stage kt+2 loads may stay in flight
        else LLMINT8_WAIT_BARRIER(0);
        if (next) read_frags(kt + 1, 0, fa[0], fb[0]);
        mfma_rows(fa[1], fb[1], 1, 4);
        __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
        __builtin_amdgcn_sched_barrier(0);
    };

    if (nk > 0) {
        // prologue: A[0], B[0] (and B[1]) in flight; wait for the first two groups
        issue_a(0);
        issue_b(0);
        if (nk > 1) {
            if (kLeadA) issue_a(1);
            else issue_b(1);
            LLMINT8_WAIT_BARRIER(4);
        } else {
            LLMINT8_WAIT_BARRIER(0);
        }
        read_frags(0, 0, fa[0], fb[0]);
        int kt = 0;
        for (; kt + 2 < nk; ++kt) stage(kt, std::true_type{});
        for (; kt < nk; ++kt) stage(kt, std::false_type{});
    }

    // ---- 16-bit outlier product and epilogue, one 32-row slice at a time
    // (lane holds column lane%32 and rows 8*(e/4) + 4*(lane/32) + e%4, e = 0..15, of each
    // 32 x 32 tile)
    const int32_t nO = *p.n_out;
    const int nsub = (nO + 15) >> 4;  // 16-deep MFMA steps over the padded outlier columns
    const int64_t wm0 = m0 + wm * 128, wn0 = n0 + wn * (32 * NJ);
    auto outlier_product = [&](const uint16_t* xo, int64_t n) {
        const int64_t bn = n < p.N ? n : p.N - 1;
        const uint16_t* wo = p.WO + bn * p.wo_pitch + h * 8;
        v16f F = v16f{};
        for (int ch = 0; ch < nsub; ++ch)
            F = mfma16<DT>(*(const u32x4*)(xo + ch * 16), *(const u32x4*)(wo + ch * 16), F);
        return F;
    };
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
                const v16f F = outlier_product(xo, n);
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
        // Every global read of the epilogue is issued first, together, so that their latencies
        // overlap (and the wait for the last operand loads): this thread's entry of the
        // factor tables and the first 16 outlier columns of the wave's rows and columns.
        const int64_t fm = m0 + tid, fn = n0 + tid - BM;
        const float sc = tid < BM ? (fm < p.M ? p.s_x[fm] : 0.0f) : (fn < p.N ? p.s_w[fn] : 0.0f);
        u32x4 xo0[4], wo0[NJ];
        if (nsub > 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t am = wm0 + 32 * i + rl < p.M ? wm0 + 32 * i + rl : p.M - 1;
                xo0[i] = *(const u32x4*)(p.XO + am * p.xo_pitch + h * 8);
            }
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int64_t bn = wn0 + 32 * j + rl < p.N ? wn0 + 32 * j + rl : p.N - 1;
                wo0[j] = *(const u32x4*)(p.WO + bn * p.wo_pitch + h * 8);
            }
        }
        // The operand slots are free once every wave is past its last reads and no load is in
        // flight: the LDS then holds the tile's dequantization factors and, per wave, its
        // 128 x 64 outputs, which leave as 16-byte row segments (full lines).
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        float* rsc = (float*)smem;  // r_i = s_x[i]/127 of the tile's rows
        float* csc = rsc + BM;      // c_n = s_w[n]/127 of its columns
        if (tid < BM) rsc[tid] = sc / 127.0f;
        else csc[tid - BM] = sc / 127.0f;
        __syncthreads();
        uint16_t* ys = (uint16_t*)(smem + kScaleBytes + w * kYStageBytes);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rb = wm * 128 + 32 * i + 4 * h;  // tile row of e = 0
            float r[16];
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const v4f t = *(const v4f*)(rsc + rb + 8 * a);
#pragma unroll
                for (int b = 0; b < 4; ++b) r[4 * a + b] = t[b];
            }
            int64_t am = wm0 + 32 * i + rl;
            am = am < p.M ? am : p.M - 1;
            const uint16_t* xo = p.XO + am * p.xo_pitch + h * 8;
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                v16f F = v16f{};
                if (nsub > 0) {
                    F = mfma16<DT>(xo0[i], wo0[j], F);
                    const int64_t n = wn0 + 32 * j + rl;
                    const uint16_t* wo = p.WO + (n < p.N ? n : p.N - 1) * p.wo_pitch + h * 8;
                    for (int ch = 1; ch < nsub; ++ch)
                        F = mfma16<DT>(*(const u32x4*)(xo + ch * 16), *(const u32x4*)(wo + ch * 16), F);
                }
                const float c = csc[wn * (32 * NJ) + 32 * j + rl];
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const float yi = __fmul_rn(__fmul_rn((float)acc[i][j][e], r[e]), c);
                    const float y = __fadd_rn(yi, p.f_scaled ? __fmul_rn(c, F[e]) : F[e]);
                    ys[(32 * i + 8 * (e >> 2) + 4 * h + (e & 3)) * kYPitch + 32 * j + rl] = from_f32<DT>(y);
                }
            }
        }
        // read back the wave's own rows (one wave's LDS accesses complete in order)
#pragma unroll 4
        for (int it = 0; it < 16; ++it) {
            const int row = it * 8 + (lane >> 3), ch = lane & 7;
            const u32x4 v = *(const u32x4*)(ys + row * kYPitch + ch * 8);
            const int64_t m = wm0 + row, n = wn0 + ch * 8;
            if (m < p.M && n < p.N) *(u32x4*)(p.Y + m * p.N + n) = v;
        }
    }
}

template <int DT, bool ACC_OUT>
hipError_t launch_one(const Params& p, hipStream_t stream) {
    const unsigned grid = (unsigned)(p.tiles_m * p.tiles_n);
    gemm_kernel<DT, ACC_OUT><<<grid, 64 * kWaves, 0, stream>>>(p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream) {
    if (a.M == 0 || a.N == 0) return hipSuccess;
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
    const bool acc_out = a.Y == nullptr;
    if (a.dt == F16) return acc_out ? launch_one<F16, true>(p, stream) : launch_one<F16, false>(p, stream);
    return acc_out ? launch_one<BF16, true>(p, stream) : launch_one<BF16, false>(p, stream);
}

}  // namespace llmint8
