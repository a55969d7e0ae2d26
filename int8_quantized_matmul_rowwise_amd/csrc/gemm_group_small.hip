// Group-wise products for a small batch (M <= 64 rows, at most 64 groups): the split-N
// layout of the vector-wise small-batch kernel -- each workgroup streams its 16 rows of Wq
// (output columns) straight from HBM into registers -- with the group-wise epilogue of the
// tiled group kernel.  The groups are taken in ascending order by the whole workgroup:
// its 4 waves split a group's 64-deep K steps (wave w: steps w, w + 4, ...), the four
// int32 partials of the group are summed exactly through LDS, and one wave per 16-row
// group folds the sum into its fp32 accumulators,
//   acc = RN32(acc + RN32(RN32((float)C_g * r_ig) * c_ng)),
// in the same op order as the tiled kernel, so both give the same bits.  Loads run in
// batches of U steps, the next batch (possibly the next group's first) issued before the
// current one's MFMAs and before the group's barrier; the LDS partials alternate between
// two buffers, so one barrier per group suffices.  The row factors r (precomputed by the
// X pass) and the column factors c = RN32(s_w / 127) of the workgroup are staged in LDS
// once.  (Group-wise scales: the "nuQmm" report page, on quantization granularity.)
#include "common.hpp"
#include "launch.hpp"

namespace llmint8 {

namespace {

constexpr int kGsWaves = 4;
constexpr int kGsMaxGroups = 64;

struct GroupSmallParams {
    const int8_t* Xq;   // M x K (pitch K)
    const int8_t* Xqb;  // NULL, or the blocked copy of Xq (xqb_offset)
    const float* rg;   // ng x M, group-major
    const int8_t* Wq;  // N x K
    const float* s_w;  // N x ng
    int64_t M, N, K;
    int G, ng;
    uint16_t* Y;
};

template <int DT, int MG>
__global__ __launch_bounds__(256) void gemm_group_small_kernel(GroupSmallParams p) {
    constexpr int U = 4;  // steps per batch and wave
    __shared__ v4i red[2][kGsWaves][MG][64];
    __shared__ float rl[kGsMaxGroups * 16 * MG];  // r[g][row]
    __shared__ float cl[kGsMaxGroups * 16];       // c[g][column]
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 15, q = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * 16;
    const int64_t n = n0 + li < p.N ? n0 + li : p.N - 1;
    const int8_t* brow = p.Wq + n * p.K;
    // lane's X row: its bytes of step st (of K) at arow[g] + (st << ash) + 16 q, row by row
    // or in the blocked copy (one 1 KB block per step and row group)
    const int8_t* arow[MG];
    const int ash = p.Xqb ? 10 : 6;
#pragma unroll
    for (int g = 0; g < MG; ++g) {
        const int64_t m = g * 16 + li < p.M ? g * 16 + li : p.M - 1;
        arow[g] = p.Xqb ? p.Xqb + xqb_offset(m, 0, p.K / 64) : p.Xq + m * p.K;
    }
    const int ng = p.ng, spg = p.G / 64;
    // the factors (ordered before their first use by the first group's barrier)
    for (int i = tid; i < ng * 16 * MG; i += 256) {
        const int g = i / (16 * MG), r = i % (16 * MG);
        rl[i] = r < p.M ? p.rg[(int64_t)g * p.M + r] : 0.0f;
    }
    for (int i = tid; i < ng * 16; i += 256) {
        const int g = i / 16, c = i % 16;
        cl[i] = n0 + c < p.N ? p.s_w[(n0 + c) * ng + g] / 127.0f : 0.0f;
    }

    // batch (g, s0): this wave's steps s0, s0 + 4, ..., s0 + 4 (U - 1) of group g (steps
    // past the group's end contribute zeros)
    auto load = [&](int g, int s0, v4i (&b)[U], v4i (&a)[U][MG]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int s = s0 + 4 * u;
            const bool in = s < spg;
            const int64_t st = (int64_t)g * spg + s;
            const int64_t k = st * 64 + q * 16;
            b[u] = in ? *(const v4i*)(brow + k) : v4i{0, 0, 0, 0};
#pragma unroll
            for (int m = 0; m < MG; ++m) a[u][m] = in ? *(const v4i*)(arow[m] + (st << ash) + q * 16) : v4i{0, 0, 0, 0};
        }
    };
    v4i acc[MG];
#pragma unroll
    for (int m = 0; m < MG; ++m) acc[m] = v4i{0, 0, 0, 0};
    auto compute = [&](const v4i (&b)[U], const v4i (&a)[U][MG]) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int m = 0; m < MG; ++m) acc[m] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[u][m], b[u], acc[m], 0, 0, 0);
    };
    v4f accf = {0.f, 0.f, 0.f, 0.f};  // waves w < MG: rows 16w + 4q + e, column li
    // end of group g: partials to LDS, barrier, fold
    auto finish_group = [&](int g) {
#pragma unroll
        for (int m = 0; m < MG; ++m) {
            red[g & 1][w][m][lane] = acc[m];
            acc[m] = v4i{0, 0, 0, 0};
        }
        __syncthreads();
        if (w < MG) {
            v4i c = red[g & 1][0][w][lane];
#pragma unroll
            for (int i = 1; i < kGsWaves; ++i) c += red[g & 1][i][w][lane];
            const float cn = cl[g * 16 + li];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float r = rl[g * 16 * MG + 16 * w + 4 * q + e];
                accf[e] = __fadd_rn(accf[e], __fmul_rn(__fmul_rn((float)c[e], r), cn));
            }
        }
    };

    {
        v4i b0[U], a0[U][MG], b1[U], a1[U][MG];
        int g = 0, s0 = w;
        load(g, s0, b0, a0);
        for (;;) {
            // the batch after (g, s0): the next steps of this group, else the next group's first
            int g1 = g, s1 = s0 + 4 * U;
            if (s1 >= spg) {
                g1 = g + 1;
                s1 = w;
            }
            if (g1 < ng) load(g1, s1, b1, a1);
            compute(b0, a0);
            if (g1 != g) finish_group(g);
            if (g1 >= ng) break;
            g = g1;
            s0 = s1;
            // the same with the buffers' roles swapped
            g1 = g;
            s1 = s0 + 4 * U;
            if (s1 >= spg) {
                g1 = g + 1;
                s1 = w;
            }
            if (g1 < ng) load(g1, s1, b0, a0);
            compute(b1, a1);
            if (g1 != g) finish_group(g);
            if (g1 >= ng) break;
            g = g1;
            s0 = s1;
        }
    }
    if (w >= MG || n0 + li >= p.N) return;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int64_t m = 16 * w + 4 * q + e;
        if (m < p.M) p.Y[m * p.N + n] = from_f32<DT>(accf[e]);
    }
}

}  // namespace

bool group_small_batch(int64_t M, int64_t K, int64_t N, int64_t G) {
    return M <= 64 && K / G <= kGsMaxGroups && small_batch(M, K, N);
}

// Measured on the 8192 x 8192 weight (cold steps, interleaved on one box), blocked against
// row by row: G = 1024 24.3 against 27.1 us at M = 16 and 38.7 against 50.1 us at M = 64;
// G = 512 26.1 / 27.3 and 42.0 / 53.4; G = 256 33.9 / 33.8 and 53.1 / 57.1; G = 128 at
// M = 16 54.5 against 53.5 us (its two steps per group make the kernel bound by the
// per-group barrier and fold, not by the operand loads).
bool group_blocked_codes(int64_t M, int64_t K, int64_t G) {
    return small_blocked_codes(M) && M <= 64 && K > 0 && G >= 256 && G <= 1024 && K / G <= kGsMaxGroups;
}

hipError_t launch_gemm_group_small(int dt, const int8_t* Xq, const int8_t* Xqb, const float* rg, const int8_t* Wq,
                                   const float* s_w, int64_t M, int64_t N, int64_t K, int64_t G, void* Y,
                                   hipStream_t stream) {
    if (M == 0 || N == 0) return hipSuccess;
    GroupSmallParams p;
    p.Xq = Xq;
    p.Xqb = Xqb;
    p.rg = rg;
    p.Wq = Wq;
    p.s_w = s_w;
    p.M = M;
    p.N = N;
    p.K = K;
    p.G = (int)G;
    p.ng = (int)(K / G);
    p.Y = (uint16_t*)Y;
    const unsigned grid = (unsigned)ceil_div(N, 16);
    const int64_t mg = ceil_div(M, 16);
#define LLMINT8_GS_LAUNCH(T)                                                                 \
    switch (mg) {                                                                            \
        case 1: gemm_group_small_kernel<T, 1><<<grid, 256, 0, stream>>>(p); break;           \
        case 2: gemm_group_small_kernel<T, 2><<<grid, 256, 0, stream>>>(p); break;           \
        case 3: gemm_group_small_kernel<T, 3><<<grid, 256, 0, stream>>>(p); break;           \
        default: gemm_group_small_kernel<T, 4><<<grid, 256, 0, stream>>>(p); break;          \
    }
    if (dt == F16) {
        LLMINT8_GS_LAUNCH(F16)
    } else {
        LLMINT8_GS_LAUNCH(BF16)
    }
#undef LLMINT8_GS_LAUNCH
    return hipGetLastError();
}

}  // namespace llmint8
