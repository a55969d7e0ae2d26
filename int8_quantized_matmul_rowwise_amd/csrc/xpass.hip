// The X pass of the LLM.int8() matmul: outlier feature dimensions, row scales, int8
// codes with the outlier columns zeroed, and the compact 16-bit outlier operands.
//
// "LLM.int8(): 8-bit Matrix Multiplication for Transformers at Scale", abstract:
// vector-wise quantization (one constant per row of X) plus a decomposition that
// isolates the outlier feature dimensions into a 16-bit product.  The outlier set is
// a property of the whole batch (talk summary "llama3-model-quantization",
// "Understanding Outliers in Transformer Models": the outliers sit in specific columns
// of the input batch), so no row can be coded before every row has been scanned: the
// pass is two HBM sweeps over X (detect, then code) around a one-workgroup compaction.
#include "common.hpp"
#include "launch.hpp"

namespace llmint8 {

// ---------------------------------------------------------------------------
// Detect: bit j of word w of partial[rb] is set iff some row of row-block rb has
// |X[i, 32w + j]| > tau.  One thread owns 8 consecutive columns (one 16-byte load per
// row); the four waves of a block split the rows.  No atomics and no pre-zeroed
// memory: every (row-block, word) slot is written exactly once.
template <int DT>
__global__ __launch_bounds__(256) void detect_kernel(const uint16_t* __restrict__ X, int64_t M, int64_t K,
                                                     int64_t rows_per_block, float tau,
                                                     uint32_t* __restrict__ partial, int64_t Kw) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t chunk = (int64_t)blockIdx.x * 64 + lane;
    const int64_t nchunks = K / 8;
    const int64_t r0 = (int64_t)blockIdx.y * rows_per_block;
    const int64_t r1 = r0 + rows_per_block < M ? r0 + rows_per_block : M;
    uint32_t mask = 0;
    if (chunk < nchunks) {
        const uint16_t* col = X + chunk * 8;
        int64_t r = r0 + w;
        for (; r + 28 < r1; r += 32) {  // eight rows in flight per thread
            u32x4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = *(const u32x4*)(col + (r + 4 * u) * K);
#pragma unroll
            for (int u = 0; u < 8; ++u)
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    uint16_t h = (uint16_t)(v[u][j >> 1] >> (16 * (j & 1)));
                    mask |= (__builtin_fabsf(to_f32<DT>(h)) > tau ? 1u : 0u) << j;
                }
        }
        for (; r < r1; r += 4) {
            u32x4 v = *(const u32x4*)(col + r * K);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                uint16_t h = (uint16_t)(v[j >> 1] >> (16 * (j & 1)));
                mask |= (__builtin_fabsf(to_f32<DT>(h)) > tau ? 1u : 0u) << j;
            }
        }
    }
    __shared__ uint32_t sm[4][64];
    sm[w][lane] = mask;
    __syncthreads();
    if (w == 0) {
        mask = sm[0][lane] | sm[1][lane] | sm[2][lane] | sm[3][lane];
        uint32_t word = mask << (8 * (lane & 3));
        word |= __shfl_xor(word, 1, kWave);
        word |= __shfl_xor(word, 2, kWave);
        const int64_t wi = chunk >> 2;
        if ((lane & 3) == 0 && wi < Kw) partial[(int64_t)blockIdx.y * Kw + wi] = word;
    }
}

// ---------------------------------------------------------------------------
// Compact (one workgroup of 1024 threads): OR the row-block partials into an LDS bitmap
// (coalesced, independent loads; LDS atomics), store the bitmap, then list the set bits in
// ascending column order (block-wide exclusive scan of per-word popcounts), and store n_O.
constexpr int64_t kMaxKw = (133143 + 31) / 32 + 1;

__global__ __launch_bounds__(1024) void compact_kernel(const uint32_t* __restrict__ partial, int64_t n_rb, int64_t Kw,
                                                       uint32_t* __restrict__ bitmap, int32_t* __restrict__ O,
                                                       int32_t* __restrict__ n_out) {
    __shared__ uint32_t bits[kMaxKw];
    __shared__ int32_t wsum[16];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    for (int64_t w = tid; w < Kw; w += 1024) bits[w] = 0;
    __syncthreads();
    const int64_t total_entries = n_rb * Kw;
    for (int64_t e0 = tid; e0 < total_entries; e0 += 8 * 1024) {
        uint32_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int64_t e = e0 + (int64_t)u * 1024;
            v[u] = e < total_entries ? partial[e] : 0u;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int64_t e = e0 + (int64_t)u * 1024;
            if (v[u]) atomicOr(&bits[e % Kw], v[u]);
        }
    }
    __syncthreads();
    int32_t base = 0;
    for (int64_t w0 = 0; w0 < Kw; w0 += 1024) {
        const int64_t wi = w0 + tid;
        const uint32_t word = wi < Kw ? bits[wi] : 0u;
        if (wi < Kw) bitmap[wi] = word;
        const int32_t cnt = __popc(word);
        int32_t incl = cnt;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int32_t t = __shfl_up(incl, off, kWave);
            if (lane >= off) incl += t;
        }
        if (lane == 63) wsum[wv] = incl;
        __syncthreads();
        int32_t before = 0, total = 0;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int32_t sq = wsum[q];
            before += q < wv ? sq : 0;
            total += sq;
        }
        int32_t pos = base + before + incl - cnt;
        uint32_t wd = word;
        while (wd) {
            const int b = __ffs(wd) - 1;
            O[pos++] = (int32_t)(wi * 32 + b);
            wd &= wd - 1;
        }
        base += total;
        __syncthreads();  // wsum is reused by the next chunk of words
    }
    if (tid == 0) *n_out = base;
}

// ---------------------------------------------------------------------------

int64_t detect_row_blocks(int64_t M) {
    if (M <= 0) return 0;
    int64_t nrb = ceil_div(M, 64);
    return nrb > 32 ? 32 : nrb;
}

hipError_t launch_detect(int dt, const void* X, int64_t M, int64_t K, float tau, uint32_t* partial,
                         hipStream_t stream) {
    const int64_t nrb = detect_row_blocks(M);
    const int64_t Kw = ceil_div(K, 32);
    if (nrb == 0 || K == 0) return hipSuccess;
    const int64_t rpb = round_up(ceil_div(M, nrb), 4);
    dim3 grid((unsigned)ceil_div(K / 8, 64), (unsigned)nrb);
    if (dt == F16)
        detect_kernel<F16><<<grid, 256, 0, stream>>>((const uint16_t*)X, M, K, rpb, tau, partial, Kw);
    else
        detect_kernel<BF16><<<grid, 256, 0, stream>>>((const uint16_t*)X, M, K, rpb, tau, partial, Kw);
    return hipGetLastError();
}

hipError_t launch_compact(int64_t M, int64_t K, const uint32_t* partial, uint32_t* bitmap, int32_t* O,
                          int32_t* n_out, hipStream_t stream) {
    const int64_t nrb = detect_row_blocks(M);
    const int64_t Kw = (M > 0 && K > 0) ? ceil_div(K, 32) : 0;
    compact_kernel<<<1, 1024, 0, stream>>>(partial, nrb, Kw, bitmap, O, n_out);
    return hipGetLastError();
}

}  // namespace llmint8

// ---------------------------------------------------------------------------
// Row coding (both paths) and the small-batch detection.  A small batch (M <= kSmallM
// rows, K <= kSmallK) takes two launches: detect_direct -- one thread per 8-column chunk
// scans all M rows and writes its bits of the bitmap directly (no row blocks, hence no
// partials and no compaction launch) -- then code_rows, whose workgroup 0 also writes O
// and n_O.  The tiled path runs detect (row-block partials), compact, then code_rows.
namespace llmint8 {

constexpr int kHold = 16;  // 16-byte chunks per thread held in registers (256 threads: K <= 32768)

template <int DT>
__global__ __launch_bounds__(256) void detect_direct_kernel(const uint16_t* __restrict__ X, int64_t M, int64_t K,
                                                            float tau, uint32_t* __restrict__ bitmap) {
    const int lane = threadIdx.x & 63;
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;  // 8-column chunk
    const int64_t nch = K / 8;
    uint32_t mask = 0;
    if (c < nch) {
        const uint16_t* col = X + c * 8;
        int64_t r = 0;
        for (; r + 8 <= M; r += 8) {
            u32x4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = *(const u32x4*)(col + (r + u) * K);
#pragma unroll
            for (int u = 0; u < 8; ++u)
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    mask |= (__builtin_fabsf(to_f32<DT>((uint16_t)(v[u][j >> 1] >> (16 * (j & 1))))) > tau ? 1u : 0u) << j;
        }
        for (; r < M; ++r) {
            const u32x4 v = *(const u32x4*)(col + r * K);
#pragma unroll
            for (int j = 0; j < 8; ++j)
                mask |= (__builtin_fabsf(to_f32<DT>((uint16_t)(v[j >> 1] >> (16 * (j & 1))))) > tau ? 1u : 0u) << j;
        }
    }
    uint32_t word = mask << (8 * (lane & 3));
    word |= __shfl_xor(word, 1, kWave);
    word |= __shfl_xor(word, 2, kWave);
    if ((lane & 3) == 0 && c < nch) bitmap[c >> 2] = word;  // K % 16 == 0: a word's chunks exist together
}

// Code the rows: workgroup i < M takes row i.  s_x[i] = max over the non-outlier columns
// of |X[i,j]|; Xq[i,j] = 0 for j in O, else the vector-wise code; Xq[i, K..pitch) = 0;
// XO[i,t] = X[i, O[t]] for t < n_O, 0 up to the next multiple of 32 (the rank t of column j
// comes from a block-wide scan of the bitmap's popcounts).  HOLD: the row stays in
// registers between the max and the coding (K <= 32768), else it is read twice.
// Workgroups M.. gather WO[n,t] = (dtype) Wq[n, O[t]] (exact; same padding), 64 rows of Wq
// each, from the O written by the compaction.  WRITE_O: workgroup 0 writes O and n_O (the
// small-batch path has no compaction launch).
template <int DT, bool HOLD, bool WRITE_O>
__global__ __launch_bounds__(256) void code_rows_kernel(const uint16_t* __restrict__ X, int64_t M, int64_t K,
                                                        const uint32_t* __restrict__ bitmap, int32_t* __restrict__ O,
                                                        int32_t* __restrict__ n_out, int8_t* __restrict__ Xq,
                                                        int64_t xq_pitch, float* __restrict__ s_x,
                                                        uint16_t* __restrict__ XO, int64_t xo_pitch,
                                                        const int8_t* __restrict__ Wq, int64_t N,
                                                        uint16_t* __restrict__ WO) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    if ((int64_t)blockIdx.x >= M) {
        const int32_t nO = *n_out;
        const int32_t P = (nO + 31) & ~31;
        const int64_t n0 = ((int64_t)blockIdx.x - M) * 64;
        for (int64_t idx = tid; idx < 64 * (int64_t)P; idx += 256) {
            const int64_t r = idx / P, t = idx % P;
            const int64_t n = n0 + r;
            if (n < N) WO[n * xo_pitch + t] = t < nO ? from_f32<DT>((float)Wq[n * K + O[t]]) : (uint16_t)0;
        }
        return;
    }
    __shared__ uint32_t bits[kMaxKw];
    __shared__ float red[4];
    __shared__ int32_t wsum[4];
    const int64_t i = blockIdx.x;
    const int64_t nch = K / 8, Kw = ceil_div(K, 32);
    const uint16_t* row = X + i * K;
    constexpr int H = HOLD ? kHold : 1;
    u32x4 v[H];
    if constexpr (HOLD) {
#pragma unroll
        for (int h = 0; h < kHold; ++h) {
            const int64_t c = tid + 256 * h;
            v[h] = c < nch ? *(const u32x4*)(row + c * 8) : u32x4{0u, 0u, 0u, 0u};
        }
    }
    for (int64_t w = tid; w < Kw; w += 256) bits[w] = bitmap[w];
    __syncthreads();
    auto obits = [&](int64_t c) { return (bits[c >> 2] >> (8 * (c & 3))) & 0xffu; };
    auto absmax8 = [&](const u32x4& x, uint32_t o, float m) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float a = __builtin_fabsf(to_f32<DT>((uint16_t)(x[j >> 1] >> (16 * (j & 1)))));
            if (!((o >> j) & 1u)) m = fmaxf(m, a);
        }
        return m;
    };
    auto code8 = [&](const u32x4& x, uint32_t o, float inv) -> u32x2 {
        u32x2 packed = {0u, 0u};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float f = to_f32<DT>((uint16_t)(x[j >> 1] >> (16 * (j & 1))));
            const int qv = ((o >> j) & 1u) ? 0 : quantize(f, inv);
            packed[j >> 2] |= ((uint32_t)qv & 0xffu) << (8 * (j & 3));
        }
        return packed;
    };

    float m = 0.0f;
    if constexpr (HOLD) {
#pragma unroll
        for (int h = 0; h < kHold; ++h) {
            const int64_t c = tid + 256 * h;
            if (c < nch) m = absmax8(v[h], obits(c), m);
        }
    } else {
        for (int64_t c = tid; c < nch; c += 256) m = absmax8(*(const u32x4*)(row + c * 8), obits(c), m);
    }
    m = wave_max(m);
    if (lane == 0) red[wv] = m;
    __syncthreads();
    const float s = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float inv = inv_scale(s);
    int8_t* qrow = Xq + i * xq_pitch;
    if constexpr (HOLD) {
#pragma unroll
        for (int h = 0; h < kHold; ++h) {
            const int64_t c = tid + 256 * h;
            if (c < nch) *(u32x2*)(qrow + c * 8) = code8(v[h], obits(c), inv);
        }
    } else {
        for (int64_t c = tid; c < nch; c += 256) *(u32x2*)(qrow + c * 8) = code8(*(const u32x4*)(row + c * 8), obits(c), inv);
    }
    for (int64_t c = nch + tid; c < xq_pitch / 8; c += 256) *(u32x2*)(qrow + c * 8) = u32x2{0u, 0u};
    if (tid == 0) s_x[i] = s;

    // outlier gather: thread tid walks words [tid*wpt, (tid+1)*wpt); its first rank is the
    // exclusive prefix of the popcounts before them
    const int64_t wpt = ceil_div(Kw, 256);
    int32_t cnt = 0;
    for (int64_t w = tid * wpt; w < (tid + 1) * wpt && w < Kw; ++w) cnt += __popc(bits[w]);
    int32_t incl = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int32_t t = __shfl_up(incl, off, kWave);
        if (lane >= off) incl += t;
    }
    if (lane == 63) wsum[wv] = incl;
    __syncthreads();
    int32_t pos = incl - cnt, total = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        pos += q < wv ? wsum[q] : 0;
        total += wsum[q];
    }
    uint16_t* xo = XO + i * xo_pitch;
    for (int64_t w = tid * wpt; w < (tid + 1) * wpt && w < Kw; ++w) {
        uint32_t wd = bits[w];
        while (wd) {
            const int b = __ffs(wd) - 1;
            const int64_t j = w * 32 + b;
            xo[pos] = row[j];
            if (WRITE_O && i == 0) O[pos] = (int32_t)j;
            ++pos;
            wd &= wd - 1;
        }
    }
    const int32_t P = (total + 31) & ~31;
    for (int64_t t = total + tid; t < P; t += 256) xo[t] = 0;
    if (WRITE_O && i == 0 && tid == 0) *n_out = total;
}

template <int DT, bool WRITE_O>
static void code_rows_launch(unsigned grid, const XPassArgs& a, const uint32_t* bitmap, int32_t* O, int32_t* n_out,
                             hipStream_t stream) {
    if (a.K <= kSmallK)
        code_rows_kernel<DT, true, WRITE_O><<<grid, 256, 0, stream>>>(
            (const uint16_t*)a.X, a.M, a.K, bitmap, O, n_out, a.Xq, a.xq_pitch, a.s_x, (uint16_t*)a.XO, a.xo_pitch,
            a.Wq, a.N, (uint16_t*)a.WO);
    else
        code_rows_kernel<DT, false, WRITE_O><<<grid, 256, 0, stream>>>(
            (const uint16_t*)a.X, a.M, a.K, bitmap, O, n_out, a.Xq, a.xq_pitch, a.s_x, (uint16_t*)a.XO, a.xo_pitch,
            a.Wq, a.N, (uint16_t*)a.WO);
}

// Big path: after detect + compact (which wrote the bitmap, O and n_O).
hipError_t launch_code_rows(const XPassArgs& a, const uint32_t* bitmap, int32_t* O, int32_t* n_out,
                            hipStream_t stream) {
    const int64_t nblk = a.M + (a.Wq ? ceil_div(a.N, 64) : 0);
    if (nblk == 0) return hipSuccess;
    if (a.dt == F16) code_rows_launch<F16, false>((unsigned)nblk, a, bitmap, O, n_out, stream);
    else code_rows_launch<BF16, false>((unsigned)nblk, a, bitmap, O, n_out, stream);
    return hipGetLastError();
}

// Small-batch path: direct detect, then the row coding also writes O and n_O.
hipError_t launch_xpass_small(const XPassArgs& a, int32_t* O, int32_t* n_out, uint32_t* bitmap, hipStream_t stream) {
    if (a.K > 0) {
        const unsigned g1 = (unsigned)ceil_div(a.K / 8, 256);
        if (a.dt == F16) detect_direct_kernel<F16><<<g1, 256, 0, stream>>>((const uint16_t*)a.X, a.M, a.K, a.tau, bitmap);
        else detect_direct_kernel<BF16><<<g1, 256, 0, stream>>>((const uint16_t*)a.X, a.M, a.K, a.tau, bitmap);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (a.dt == F16) code_rows_launch<F16, true>((unsigned)a.M, a, bitmap, O, n_out, stream);
    else code_rows_launch<BF16, true>((unsigned)a.M, a, bitmap, O, n_out, stream);
    return hipGetLastError();
}

}  // namespace llmint8
