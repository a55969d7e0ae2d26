// Products and epilogue of the LLM.int8() matmul for a small batch (M <= 128 tokens: the
// decode shapes).  The same arithmetic as the tiled kernel (exact int32 C = Xq Wq^T on i8
// MFMA, fp32 F = X[:,O] Wq[:,O]^T on 16-bit MFMA, the same epilogue op sequence), laid
// out for an HBM-bound product: the weight is read once, so every workgroup streams its
// own 16 or 32 rows of Wq (output columns) straight from HBM into registers -- no LDS
// staging -- and the waves of a workgroup split K, each keeping two batches of K steps in
// flight (the next batch is loaded before the current one's MFMAs).  Two 64-deep steps of
// a wave cover one 128-byte line of each Wq row.  Every workgroup re-reads all of Xq from
// the cache; with 32 columns per workgroup each X operand load feeds two MFMAs, which
// halves those re-reads (they grow with M).  From 8 rows up they read the blocked copy of
// Xq that the small-batch X pass writes (xqb_offset), where one operand load is one 1 KB
// block, eight whole cache lines, instead of halves of 16 lines.  Partial int32 sums are
// combined exactly through LDS.  Each workgroup gathers the 16-bit outlier operands
// Wq[n, O[t]] of its own columns, at kernel start so that the scattered loads overlap the
// weight stream.
// "LLM.int8(): 8-bit Matrix Multiplication for Transformers at Scale", abstract.
#include "common.hpp"
#include "launch.hpp"

namespace llmint8 {

namespace {


struct SmallParams {
    const int8_t* Xq;
    int64_t xq_pitch;
    const int8_t* Xqb;  // NULL: Xq row by row; else the blocked copy (xqb_offset)
    const int8_t* Wq;
    int64_t M, N, K;
    const float* s_x;
    const float* s_w;
    const uint16_t* XO;
    int64_t xo_pitch;
    const uint16_t* WO;  // NULL: gather Wq[n, O[t]] (scaled outlier term); else exact rows
    int64_t wo_pitch;
    const int32_t* O;
    const int32_t* n_out;
    uint16_t* Y;
    int32_t* C_acc;
    float* F_acc;
};

template <int DT>
__device__ __forceinline__ v4f mfma16x16(const u32x4& a, const u32x4& b, const v4f& c) {
    if constexpr (DT == F16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, a), __builtin_bit_cast(v8h, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
}

// The W side of the outlier product for column n and outlier ranks t = t0 + 8q + e (e < 8),
// packed two per dword: the caller's exact row W_O[n, t], else (T)Wq[n, O[t]]; 0 for t >=
// n_O.  Every load is issued unconditionally (ranks past n_O read the last outlier's
// entries, then are zeroed), so the eight O loads share one round trip and the eight
// gathers the next, instead of two dependent trips per outlier.
template <int DT>
__device__ __forceinline__ void gather_w_side(const SmallParams& p, int64_t n, int t0, int q, int32_t nO,
                                              uint32_t (&out)[4]) {
    uint16_t h[8];
    if (p.WO) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int t = t0 + q * 8 + e;
            h[e] = p.WO[n * p.wo_pitch + (t < nO ? t : nO - 1)];
        }
    } else {
        int32_t col[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int t = t0 + q * 8 + e;
            col[e] = p.O[t < nO ? t : nO - 1];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = from_f32<DT>((float)p.Wq[n * p.K + col[e]]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e)
        out[e >> 1] |= (uint32_t)(t0 + q * 8 + e < nO ? h[e] : (uint16_t)0) << (16 * (e & 1));
}

// MG: groups of 16 rows of X (ceil(M/16)); NC: groups of 16 output columns per
// workgroup (each X operand load feeds NC MFMAs, so Xq is re-read from the cache N / (16
// NC) times instead of N / 16).  Batches of PAIRS step pairs per wave, two register sets:
// the next batch's loads are issued before the current batch's MFMAs, so the weight
// stream never waits for the arithmetic.  WAVES waves split K; waves g * NC + c (g < MG,
// c < NC) finish the row group g of column group c: MG * NC <= WAVES.  The one-group
// layout (decode shapes) is held to three waves per SIMD (at most 168 registers).
template <int DT, int MG, int NC, int WAVES, bool ACC_OUT>
__global__ __launch_bounds__(64 * WAVES, MG == 1 && NC == 1 ? 3 : 1) void gemm_small_kernel(SmallParams p) {
    static_assert(MG * NC <= WAVES, "one finishing wave per row and column group");
    constexpr int kWaves = WAVES;
    constexpr int PAIRS = MG == 1 ? 4 : (MG * NC == 2 ? 2 : 1);
    constexpr int U = 2 * PAIRS;  // 64-deep steps per batch
    __shared__ v4i red[kWaves][MG][NC][64];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int li = lane & 15, q = lane >> 4;  // 16x16x64 operands: row/column li, 16 k at 16*q
    const int64_t n0 = (int64_t)blockIdx.x * 16 * NC;
    const int8_t* brow[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int64_t n = n0 + 16 * c + li < p.N ? n0 + 16 * c + li : p.N - 1;
        brow[c] = p.Wq + n * p.K;
    }
    const int64_t nsteps = ceil_div(p.K, 64);
    // lane's X row: its bytes of step st at arow[g] + (st << ash) + 16 q.  Row by row the
    // rows are zero-padded up to a multiple of 256 bytes; in the blocked copy one step of a
    // row group is one 1 KB block (whole cache lines), zero past K.  Rows past M read row
    // M - 1 (their sums are not stored).
    const int8_t* arow[MG];
    const int ash = p.Xqb ? 10 : 6;
#pragma unroll
    for (int g = 0; g < MG; ++g) {
        const int64_t m = g * 16 + li < p.M ? g * 16 + li : p.M - 1;
        arow[g] = p.Xqb ? p.Xqb + xqb_offset(m, 0, nsteps) : p.Xq + m * p.xq_pitch;
    }

    // The outlier operands of the epilogue (first 32 outlier columns), gathered now so that
    // their scattered loads overlap the weight stream: for the finishing wave of (g, c),
    // Wq[n, O[t]] for t = 8q + e, and the row's X[:,O] chunk.
    const int32_t nO = *p.n_out;
    const int fg = w / NC, fc = w % NC;  // this wave's row and column group when it finishes
    const int64_t fn = n0 + 16 * fc + li < p.N ? n0 + 16 * fc + li : p.N - 1;
    uint32_t wo0[4] = {0u, 0u, 0u, 0u};
    u32x4 xo0 = {0u, 0u, 0u, 0u};
    if (w < MG * NC && nO > 0) {
        const int64_t am = fg * 16 + li < p.M ? fg * 16 + li : p.M - 1;
        xo0 = *(const u32x4*)(p.XO + am * p.xo_pitch + q * 8);
        gather_w_side<DT>(p, fn, 0, q, nO, wo0);
    }

    v4i acc[MG][NC];
#pragma unroll
    for (int g = 0; g < MG; ++g)
#pragma unroll
        for (int c = 0; c < NC; ++c) acc[g][c] = v4i{0, 0, 0, 0};
    // wave w takes step pairs w, w+4, w+8, ...; batch j of the wave holds pairs
    // w + kWaves * (PAIRS * j + i), i < PAIRS
    const int64_t stride = (int64_t)kWaves * PAIRS;
    auto load = [&](int64_t p0, v4i (&b)[U][NC], v4i (&a)[U][MG]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t st = 2 * (p0 + (int64_t)kWaves * (u >> 1)) + (u & 1);
            const int64_t k = st * 64 + q * 16;
            const bool in = st < nsteps;
#pragma unroll
            for (int c = 0; c < NC; ++c) b[u][c] = (in && k < p.K) ? *(const v4i*)(brow[c] + k) : v4i{0, 0, 0, 0};
#pragma unroll
            for (int g = 0; g < MG; ++g)
                a[u][g] = in ? *(const v4i*)(arow[g] + (st << ash) + q * 16) : v4i{0, 0, 0, 0};
        }
    };
    auto compute = [&](const v4i (&b)[U][NC], const v4i (&a)[U][MG]) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int g = 0; g < MG; ++g)
#pragma unroll
                for (int c = 0; c < NC; ++c)
                    acc[g][c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[u][g], b[u][c], acc[g][c], 0, 0, 0);
    };
    {
        v4i b0[U][NC], a0[U][MG], b1[U][NC], a1[U][MG];
        int64_t p0 = w;
        if (2 * p0 < nsteps) load(p0, b0, a0);
        while (2 * p0 < nsteps) {
            const int64_t p1 = p0 + stride;
            if (2 * p1 < nsteps) load(p1, b1, a1);
            compute(b0, a0);
            if (2 * p1 >= nsteps) break;
            const int64_t p2 = p1 + stride;
            if (2 * p2 < nsteps) load(p2, b0, a0);
            compute(b1, a1);
            p0 = p2;
        }
    }
#pragma unroll
    for (int g = 0; g < MG; ++g)
#pragma unroll
        for (int c = 0; c < NC; ++c) red[w][g][c][lane] = acc[g][c];
    __syncthreads();
    if (w >= MG * NC) return;

    // ---- wave (g, c): rows 16g.., columns n0 + 16c.., exact sum of the four partials,
    // outlier product, epilogue
    const int g = fg, c = fc;
    const int64_t n = fn;
    v4i cs = red[0][g][c][lane];
#pragma unroll
    for (int i = 1; i < kWaves; ++i) cs += red[i][g][c][lane];
    v4f F = v4f{0.f, 0.f, 0.f, 0.f};
    if (nO > 0) F = mfma16x16<DT>(xo0, u32x4{wo0[0], wo0[1], wo0[2], wo0[3]}, F);
    {
        const int64_t am = g * 16 + li < p.M ? g * 16 + li : p.M - 1;
        const uint16_t* xo = p.XO + am * p.xo_pitch + q * 8;
        for (int t0 = 32; t0 < nO; t0 += 32) {
            const u32x4 av = *(const u32x4*)(xo + t0);  // zero-padded to a multiple of 32
            uint32_t bw[4] = {0u, 0u, 0u, 0u};
            gather_w_side<DT>(p, n, t0, q, nO, bw);
            F = mfma16x16<DT>(av, u32x4{bw[0], bw[1], bw[2], bw[3]}, F);
        }
    }
    if (n0 + 16 * c + li >= p.N) return;
    const float cn = p.s_w[n] / 127.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {  // lane holds rows 4q + e of the group, column li
        const int64_t m = g * 16 + 4 * q + e;
        if (m >= p.M) continue;
        if constexpr (ACC_OUT) {
            p.C_acc[m * p.N + n] = cs[e];
            p.F_acc[m * p.N + n] = F[e];
        } else {
            const float r = p.s_x[m] / 127.0f;
            const float yi = __fmul_rn(__fmul_rn((float)cs[e], r), cn);
            const float y = __fadd_rn(yi, p.WO ? F[e] : __fmul_rn(cn, F[e]));
            p.Y[m * p.N + n] = from_f32<DT>(y);
        }
    }
}

// Up to 4 row groups: two column groups per workgroup when that still gives every compute
// unit a workgroup (and, for one row group, two: with one the single 16-column layout is
// faster), with 8 waves for 3 or 4 row groups; else one column group and 4 waves.  5 to 8
// row groups: one column group and 8 waves.  Measured on MI355X, N x K = 36864 x 12288,
// 28672 x 8192, 16384 x 4096, 14336 x 4096, 8192 x 8192 and 4096 x 4096, M = 16 to 128.
template <int DT, bool ACC_OUT>
hipError_t launch_mg(const SmallParams& p, hipStream_t stream) {
    const int64_t mg = ceil_div(p.M, 16);
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (mg > 4) {  // 65 to 128 rows: one column group, 8 waves
        const unsigned grid = (unsigned)ceil_div(p.N, 16);
        switch (mg) {
            case 5: gemm_small_kernel<DT, 5, 1, 8, ACC_OUT><<<grid, 512, 0, stream>>>(p); break;
            case 6: gemm_small_kernel<DT, 6, 1, 8, ACC_OUT><<<grid, 512, 0, stream>>>(p); break;
            case 7: gemm_small_kernel<DT, 7, 1, 8, ACC_OUT><<<grid, 512, 0, stream>>>(p); break;
            default: gemm_small_kernel<DT, 8, 1, 8, ACC_OUT><<<grid, 512, 0, stream>>>(p); break;
        }
        return hipGetLastError();
    }
    const int64_t wg2 = ceil_div(p.N, 32);
    if (wg2 >= cus && (mg > 1 || wg2 >= 2 * (int64_t)cus)) {
        const unsigned grid = (unsigned)wg2;
        switch (mg) {
            case 1: gemm_small_kernel<DT, 1, 2, 4, ACC_OUT><<<grid, 256, 0, stream>>>(p); break;
            case 2: gemm_small_kernel<DT, 2, 2, 4, ACC_OUT><<<grid, 256, 0, stream>>>(p); break;
            case 3: gemm_small_kernel<DT, 3, 2, 8, ACC_OUT><<<grid, 512, 0, stream>>>(p); break;
            default: gemm_small_kernel<DT, 4, 2, 8, ACC_OUT><<<grid, 512, 0, stream>>>(p); break;
        }
        return hipGetLastError();
    }
    const unsigned grid = (unsigned)ceil_div(p.N, 16);
    switch (mg) {
        case 1: gemm_small_kernel<DT, 1, 1, 4, ACC_OUT><<<grid, 256, 0, stream>>>(p); break;
        case 2: gemm_small_kernel<DT, 2, 1, 4, ACC_OUT><<<grid, 256, 0, stream>>>(p); break;
        case 3: gemm_small_kernel<DT, 3, 1, 4, ACC_OUT><<<grid, 256, 0, stream>>>(p); break;
        default: gemm_small_kernel<DT, 4, 1, 4, ACC_OUT><<<grid, 256, 0, stream>>>(p); break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_small(const GemmArgs& a, hipStream_t stream) {
    if (a.M == 0 || a.N == 0) return hipSuccess;
    SmallParams p;
    p.Xq = a.Xq;
    p.xq_pitch = a.xq_pitch;
    p.Xqb = a.Xqb;
    p.Wq = a.Wq;
    p.M = a.M;
    p.N = a.N;
    p.K = a.K;
    p.s_x = a.s_x;
    p.s_w = a.s_w;
    p.XO = (const uint16_t*)a.XO;
    p.xo_pitch = a.xo_pitch;
    p.WO = a.f_scaled ? nullptr : (const uint16_t*)a.WO;
    p.wo_pitch = a.wo_pitch;
    p.O = a.O;
    p.n_out = a.n_out;
    p.Y = (uint16_t*)a.Y;
    p.C_acc = a.C_acc;
    p.F_acc = a.F_acc;
    const bool acc_out = a.Y == nullptr;
    if (a.dt == F16) return acc_out ? launch_mg<F16, true>(p, stream) : launch_mg<F16, false>(p, stream);
    return acc_out ? launch_mg<BF16, true>(p, stream) : launch_mg<BF16, false>(p, stream);
}

}  // namespace llmint8
