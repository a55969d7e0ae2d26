// Products and epilogue of the LLM.int8() matmul for a small batch (M <= 64 tokens: the
// decode shape).  The same arithmetic as the tiled kernel (exact int32 C = Xq Wq^T on i8
// MFMA, fp32 F = X[:,O] Wq[:,O]^T on 16-bit MFMA, the same epilogue op sequence), laid
// out for an HBM-bound product: the weight is read once, so every workgroup streams its
// own 16 rows of Wq (16 output columns) straight from HBM into registers -- no LDS
// staging, nothing to reuse -- and the four waves of a workgroup split K, each keeping
// two batches of K steps in flight (the next batch is loaded before the current one's
// MFMAs).  Two 64-deep steps of a wave cover one 128-byte line of each Wq row.  Partial
// int32 sums are combined exactly through LDS.  Each workgroup gathers the 16-bit outlier
// operands Wq[n, O[t]] of its own columns, at kernel start so that the scattered loads
// overlap the weight stream.
// "LLM.int8(): 8-bit Matrix Multiplication for Transformers at Scale", abstract.
#include "common.hpp"
#include "launch.hpp"

namespace llmint8 {

namespace {

constexpr int kCols = 16;   // output columns per workgroup
constexpr int kWaves = 4;   // waves per workgroup, splitting K

struct SmallParams {
    const int8_t* Xq;
    int64_t xq_pitch;
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

// MG: groups of 16 rows of X (ceil(M/16)).  Batches of PAIRS step pairs per wave, two
// register sets: the next batch's loads are issued before the current batch's MFMAs, so
// the weight stream never waits for the arithmetic.
template <int DT, int MG, bool ACC_OUT>
__global__ __launch_bounds__(256) void gemm_small_kernel(SmallParams p) {
    constexpr int PAIRS = MG == 1 ? 4 : (MG == 2 ? 2 : 1);
    constexpr int U = 2 * PAIRS;  // 64-deep steps per batch
    __shared__ v4i red[kWaves][MG][64];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int li = lane & 15, q = lane >> 4;  // 16x16x64 operands: row/column li, 16 k at 16*q
    const int64_t n0 = (int64_t)blockIdx.x * kCols;
    const int64_t n = n0 + li < p.N ? n0 + li : p.N - 1;
    const int8_t* brow = p.Wq + n * p.K;
    const int8_t* arow[MG];
#pragma unroll
    for (int g = 0; g < MG; ++g) {
        const int64_t m = g * 16 + li < p.M ? g * 16 + li : p.M - 1;
        arow[g] = p.Xq + m * p.xq_pitch;  // rows are zero-padded up to a multiple of 256 bytes
    }
    const int64_t nsteps = ceil_div(p.K, 64);

    // The outlier operands of the epilogue (first 32 outlier columns), gathered now so that
    // their scattered loads overlap the weight stream: Wq[n, O[t]] for t = 8q + e, and the
    // row's X[:,O] chunk.
    const int32_t nO = *p.n_out;
    uint32_t wo0[4] = {0u, 0u, 0u, 0u};
    u32x4 xo0 = {0u, 0u, 0u, 0u};
    if (w < MG && nO > 0) {
        const int64_t am = w * 16 + li < p.M ? w * 16 + li : p.M - 1;
        xo0 = *(const u32x4*)(p.XO + am * p.xo_pitch + q * 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int t = q * 8 + e;
            const uint16_t hv = t >= nO ? (uint16_t)0
                                : p.WO ? p.WO[n * p.wo_pitch + t] : from_f32<DT>((float)brow[p.O[t]]);
            wo0[e >> 1] |= (uint32_t)hv << (16 * (e & 1));
        }
    }

    v4i acc[MG];
#pragma unroll
    for (int g = 0; g < MG; ++g) acc[g] = v4i{0, 0, 0, 0};
    // wave w takes step pairs w, w+4, w+8, ...; batch j of the wave holds pairs
    // w + kWaves * (PAIRS * j + i), i < PAIRS
    const int64_t stride = (int64_t)kWaves * PAIRS;
    auto load = [&](int64_t p0, v4i (&b)[U], v4i (&a)[U][MG]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t st = 2 * (p0 + (int64_t)kWaves * (u >> 1)) + (u & 1);
            const int64_t k = st * 64 + q * 16;
            const bool in = st < nsteps;
            b[u] = (in && k < p.K) ? *(const v4i*)(brow + k) : v4i{0, 0, 0, 0};
#pragma unroll
            for (int g = 0; g < MG; ++g) a[u][g] = in ? *(const v4i*)(arow[g] + k) : v4i{0, 0, 0, 0};
        }
    };
    auto compute = [&](const v4i (&b)[U], const v4i (&a)[U][MG]) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int g = 0; g < MG; ++g) acc[g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[u][g], b[u], acc[g], 0, 0, 0);
    };
    {
        v4i b0[U], a0[U][MG], b1[U], a1[U][MG];
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
    for (int g = 0; g < MG; ++g) red[w][g][lane] = acc[g];
    __syncthreads();
    if (w >= MG) return;

    // ---- wave g: rows 16g.., exact sum of the four partials, outlier product, epilogue
    const int g = w;
    const v4i c = red[0][g][lane] + red[1][g][lane] + red[2][g][lane] + red[3][g][lane];
    v4f F = v4f{0.f, 0.f, 0.f, 0.f};
    if (nO > 0) F = mfma16x16<DT>(xo0, u32x4{wo0[0], wo0[1], wo0[2], wo0[3]}, F);
    {
        const int64_t am = g * 16 + li < p.M ? g * 16 + li : p.M - 1;
        const uint16_t* xo = p.XO + am * p.xo_pitch + q * 8;
        for (int t0 = 32; t0 < nO; t0 += 32) {
            const u32x4 av = *(const u32x4*)(xo + t0);  // zero-padded to a multiple of 32
            u32x4 bv = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int t = t0 + q * 8 + e;
                const uint16_t h = t >= nO ? (uint16_t)0
                                   : p.WO ? p.WO[n * p.wo_pitch + t] : from_f32<DT>((float)brow[p.O[t]]);
                bv[e >> 1] |= (uint32_t)h << (16 * (e & 1));
            }
            F = mfma16x16<DT>(av, bv, F);
        }
    }
    if (n0 + li >= p.N) return;
    const float cn = p.s_w[n] / 127.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {  // lane holds rows 4q + e of the group, column li
        const int64_t m = g * 16 + 4 * q + e;
        if (m >= p.M) continue;
        if constexpr (ACC_OUT) {
            p.C_acc[m * p.N + n] = c[e];
            p.F_acc[m * p.N + n] = F[e];
        } else {
            const float r = p.s_x[m] / 127.0f;
            const float yi = __fmul_rn(__fmul_rn((float)c[e], r), cn);
            const float y = __fadd_rn(yi, p.WO ? F[e] : __fmul_rn(cn, F[e]));
            p.Y[m * p.N + n] = from_f32<DT>(y);
        }
    }
}

template <int DT, bool ACC_OUT>
hipError_t launch_mg(const SmallParams& p, hipStream_t stream) {
    const unsigned grid = (unsigned)ceil_div(p.N, kCols);
    switch (ceil_div(p.M, 16)) {
        case 1: gemm_small_kernel<DT, 1, ACC_OUT><<<grid, 256, 0, stream>>>(p); break;
        case 2: gemm_small_kernel<DT, 2, ACC_OUT><<<grid, 256, 0, stream>>>(p); break;
        case 3: gemm_small_kernel<DT, 3, ACC_OUT><<<grid, 256, 0, stream>>>(p); break;
        default: gemm_small_kernel<DT, 4, ACC_OUT><<<grid, 256, 0, stream>>>(p); break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_small(const GemmArgs& a, hipStream_t stream) {
    if (a.M == 0 || a.N == 0) return hipSuccess;
    SmallParams p;
    p.Xq = a.Xq;
    p.xq_pitch = a.xq_pitch;
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
