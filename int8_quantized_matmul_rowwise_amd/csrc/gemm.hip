// The products of the LLM.int8() matmul and its dequantizing epilogue, one kernel:
//   C = Xq Wq^T            int8 x int8 -> int32 on v_mfma_i32_16x16x64_i8 (exact),
//   F = X[:,O] Wq[:,O]^T   16-bit x 16-bit -> fp32 on v_mfma_f32_16x16x32_{f16,bf16},
//   y = RN((RN(RN((float)C * r_i) * c_n)) + RN(c_n * F)),  r_i = s_x/127, c_n = s_w/127,
//   Y = y rounded to the 16-bit type.
// "LLM.int8(): 8-bit Matrix Multiplication for Transformers at Scale", abstract: the
// int8 product with one normalization constant per inner-product vector, and the
// outlier feature dimensions through a 16-bit product, summed into the same output.
//
// Tiling (gfx950: 64-wide waves, 160 KB LDS, 512 registers per lane at one wave/SIMD):
//   block tile 256 x 256, K step 128 bytes, 4 waves in 2 x 2, each wave 128 x 128 =
//   8 x 8 MFMA tiles of 16 x 16 -> 256 int32 accumulators per lane.
//   Operands go HBM/L2 -> LDS with global_load_lds (16 B per lane, no register
//   staging), two stages of 64 KB.  LDS rows are 128 B; the 16-byte chunk c of row r
//   is stored at chunk c ^ (r & 7) ^ ((r >> 3) & 1), so the ds_read_b128 of 16
//   consecutive rows at one k hit distinct banks.
//   Tiles are assigned so that the workgroups the dispatcher places on one XCD (ids
//   congruent mod 8) take a contiguous run of tiles in grouped order (4 row-tiles per
//   group): concurrently running tiles on an XCD share A and B panels in its L2.
#include "common.hpp"
#include "launch.hpp"

namespace llmint8 {

namespace {

constexpr int BM = 256, BN = 256, BK = 128;
constexpr int kStageBytes = (BM + BN) * BK;  // 64 KB
constexpr int kStages = 2;
constexpr int kGroupM = 4;
constexpr int kXcds = 8;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ void load_lds16(const void* g, int8_t* lds_base) {
    __builtin_amdgcn_global_load_lds(g, (lds_ptr_t)lds_base, 16, 0, 0);
}

struct Params {
    const int8_t* Xq;
    int64_t xq_pitch;
    const int8_t* Wq;
    int64_t M, N, K;
    const float* s_x;
    const float* s_w;
    const uint16_t* XO;
    const uint16_t* WO;
    int64_t xo_pitch;
    const int32_t* n_out;
    uint16_t* Y;
    int32_t* C_acc;
    float* F_acc;
    int tiles_m, tiles_n;
};

template <int DT>
__device__ __forceinline__ v4f mfma16(const u32x4& a, const u32x4& b, const v4f& c) {
    if constexpr (DT == F16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, a), __builtin_bit_cast(v8h, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
}

template <int DT, bool ACC_OUT>
__global__ __launch_bounds__(256, 1) void gemm_kernel(Params p) {
    __shared__ __attribute__((aligned(1024))) int8_t smem[kStages * kStageBytes];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w >> 1, wn = w & 1;

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

    // ---- loader: wave w fills LDS slots [64*(8w+j), +64) of each operand, j = 0..7:
    // rows r = 64w + 8j + lane/8, physical chunk lane%8 -> logical chunk c.
    const int lrow = 64 * w + (lane >> 3);
    const int c_even = (lane & 7) ^ (lane >> 3);      // j even: (r>>3)&1 == 0
    const int c_odd = c_even ^ 1;                     // j odd
    const int nk = (int)ceil_div(p.K, BK);

    auto issue_stage = [&](int kt, int stage) {
        int8_t* As = smem + stage * kStageBytes;
        int8_t* Bs = As + BM * BK;
        const int64_t kb = (int64_t)kt * BK;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int r = lrow + 8 * j;
            const int c = (j & 1) ? c_odd : c_even;
            int64_t m = m0 + r;
            m = m < p.M ? m : p.M - 1;
            load_lds16(p.Xq + m * p.xq_pitch + kb + c * 16, As + (8 * w + j) * 1024);
            int64_t n = n0 + r;
            n = n < p.N ? n : p.N - 1;
            int64_t k = kb + c * 16;
            k = k < p.K ? k : 0;  // past K the A side is zero; any in-bounds bytes will do
            load_lds16(p.Wq + n * p.K + k, Bs + (8 * w + j) * 1024);
        }
    };

    // ---- per-lane LDS read offsets for the MFMA operands (row within the wave's
    // 128-row panel: 16*bi + lane%16; k chunk 4*ks + lane/16)
    const int s = (lane & 7) ^ ((lane >> 3) & 1);
    const int q = lane >> 4;
    const int rd0 = (lane & 15) * BK + ((q ^ s) << 4);
    const int rd1 = (lane & 15) * BK + (((q + 4) ^ s) << 4);

    v4i acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = v4i{0, 0, 0, 0};

    if (nk > 0) issue_stage(0, 0);
    for (int kt = 0; kt < nk; ++kt) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (kt + 1 < nk) issue_stage(kt + 1, (kt + 1) & 1);
        const int8_t* As = smem + (kt & 1) * kStageBytes + wm * 128 * BK;
        const int8_t* Bs = smem + (kt & 1) * kStageBytes + BM * BK + wn * 128 * BK;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int rd = ks ? rd1 : rd0;
            v4i a[8], b[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) a[i] = *(const v4i*)(As + rd + i * 16 * BK);
#pragma unroll
            for (int j = 0; j < 8; ++j) b[j] = *(const v4i*)(Bs + rd + j * 16 * BK);
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    }

    // ---- 16-bit outlier product and epilogue, one 16-row slice at a time
    const int32_t nO = *p.n_out;
    const int nchunk = (nO + 31) >> 5;
    const int64_t wm0 = m0 + wm * 128, wn0 = n0 + wn * 128;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        v4f F[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) F[j] = v4f{0.f, 0.f, 0.f, 0.f};
        for (int ch = 0; ch < nchunk; ++ch) {
            int64_t am = wm0 + 16 * i + (lane & 15);
            am = am < p.M ? am : p.M - 1;
            const u32x4 a = *(const u32x4*)(p.XO + am * p.xo_pitch + ch * 32 + q * 8);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                int64_t bn = wn0 + 16 * j + (lane & 15);
                bn = bn < p.N ? bn : p.N - 1;
                const u32x4 b = *(const u32x4*)(p.WO + bn * p.xo_pitch + ch * 32 + q * 8);
                F[j] = mfma16<DT>(a, b, F[j]);
            }
        }
        // lane holds rows 16i + 4q + e (e = 0..3) and column lane%16 of each 16x16 tile
        float r[4];
        int64_t mrow[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            mrow[e] = wm0 + 16 * i + 4 * q + e;
            r[e] = mrow[e] < p.M ? p.s_x[mrow[e]] / 127.0f : 0.0f;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int64_t n = wn0 + 16 * j + (lane & 15);
            if (n >= p.N) continue;
            const float c = p.s_w[n] / 127.0f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (mrow[e] >= p.M) continue;
                if constexpr (ACC_OUT) {
                    p.C_acc[mrow[e] * p.N + n] = acc[i][j][e];
                    p.F_acc[mrow[e] * p.N + n] = F[j][e];
                } else {
                    const float yi = __fmul_rn(__fmul_rn((float)acc[i][j][e], r[e]), c);
                    const float y = __fadd_rn(yi, __fmul_rn(c, F[j][e]));
                    p.Y[mrow[e] * p.N + n] = from_f32<DT>(y);
                }
            }
        }
    }
}

template <int DT, bool ACC_OUT>
hipError_t launch_one(const Params& p, hipStream_t stream) {
    const unsigned grid = (unsigned)(p.tiles_m * p.tiles_n);
    gemm_kernel<DT, ACC_OUT><<<grid, 256, 0, stream>>>(p);
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
