// Offline weight conversion: column absmax scales and the int8 codes of W, stored
// transposed (N x K, each output column's codes contiguous) for the int8 product.
//
// "LLM.int8(): 8-bit Matrix Multiplication for Transformers at Scale", abstract: a
// 16-bit checkpoint is loaded, converted to Int8 and used immediately (one data-free
// pass; round to nearest -- "nuQmm" report page, GPTQ statements under
// "Large-model Quantization" and "The Gptq Algorithm").  One normalization constant
// per output column of W: its absmax.  With a fixed outlier set (skip: a bitmap over the
// rows of W), those rows are left out of the scale, coded 0, and copied exactly into the
// 16-bit W_O (N x P) by gather_wo_kernel.
#include "common.hpp"
#include "launch.hpp"

namespace llmint8 {

__global__ void fill_zero_kernel(float* __restrict__ p, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0.0f;
}

// s_w[n] = max_k |W[k,n]|: each block reduces a 512-column x (K/splits)-row slab and
// merges with atomicMax on the fp32 bit pattern (|w| >= 0, so the unsigned order of
// the bits is the numeric order: exact and independent of the merge order).
__device__ __forceinline__ bool skipped(const uint32_t* skip, int64_t k) {
    return skip && ((skip[k >> 5] >> (k & 31)) & 1u);
}

template <int DT>
__global__ __launch_bounds__(256) void colmax_kernel(const uint16_t* __restrict__ W, int64_t K, int64_t N,
                                                     int64_t rows_per_split, const uint32_t* __restrict__ skip,
                                                     float* __restrict__ s_w) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t n8 = ((int64_t)blockIdx.x * 64 + lane) * 8;
    const int64_t k0 = (int64_t)blockIdx.y * rows_per_split;
    const int64_t k1 = k0 + rows_per_split < K ? k0 + rows_per_split : K;
    float m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (n8 < N) {
        for (int64_t k = k0 + w; k < k1; k += 4) {
            if (skipped(skip, k)) continue;  // the same row for the whole wave
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
        for (int j = 0; j < 8; ++j) {
            const float r = fmaxf(fmaxf(sm[0][lane][j], sm[1][lane][j]), fmaxf(sm[2][lane][j], sm[3][lane][j]));
            atomicMax((unsigned int*)(s_w + n8 + j), __float_as_uint(r));
        }
    }
}

// Wq[n,k] = code of W[k,n] with the column's scale.  Tile: 128 rows of W (k) x 64
// columns (n); read along n (coalesced), transpose through LDS, write along k.  Scales
// per group of G rows (G a multiple of 128, so a tile lies in one group): the scale of
// column n and group g is s_w[n*ng + g]; the vector-wise case is ng = 1, G = K.
template <int DT>
__global__ __launch_bounds__(256) void quantize_weight_kernel(const uint16_t* __restrict__ W, int64_t K, int64_t N,
                                                              const float* __restrict__ s_w, int64_t ng, int64_t G,
                                                              const uint32_t* __restrict__ skip,
                                                              int8_t* __restrict__ Wq) {
    __shared__ float inv[64];
    __shared__ __attribute__((aligned(16))) uint8_t tile[64][128 + 16];
    const int tid = threadIdx.x;
    const int64_t n0 = (int64_t)blockIdx.x * 64, k0 = (int64_t)blockIdx.y * 128;
    if (tid < 64) inv[tid] = (n0 + tid < N) ? inv_scale(s_w[(n0 + tid) * ng + k0 / G]) : 0.0f;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int q = tid + 256 * u;
        const int kk = q >> 3, cc = q & 7;
        const int64_t k = k0 + kk, n = n0 + cc * 8;
        if (k < K && n < N) {
            const u32x4 v = *(const u32x4*)(W + k * N + n);
            const bool out = skipped(skip, k);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float f = to_f32<DT>((uint16_t)(v[j >> 1] >> (16 * (j & 1))));
                tile[cc * 8 + j][kk] = out ? (uint8_t)0 : (uint8_t)quantize(f, inv[cc * 8 + j]);
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int q = tid + 256 * u;
        const int nl = q >> 3, kc = q & 7;
        const int64_t n = n0 + nl, k = k0 + kc * 16;
        if (n < N && k < K) *(u32x4*)(Wq + n * K + k) = *(const u32x4*)(&tile[nl][kc * 16]);
    }
}

// W_O[n, t] = W[O[t], n] (exact), zero for t >= n_O up to the pitch P; entries of O
// outside [0, K) give zero (never an access outside W).
__global__ __launch_bounds__(256) void gather_wo_kernel(const uint16_t* __restrict__ W, int64_t K, int64_t N,
                                                        const int32_t* __restrict__ O, int64_t nO, int64_t P,
                                                        uint16_t* __restrict__ WO) {
    const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (n >= N) return;
    for (int64_t t = blockIdx.y; t < P; t += gridDim.y) {  // grid.y is capped at 65535
        const int64_t k = t < nO ? (int64_t)O[t] : -1;
        WO[n * P + t] = (k >= 0 && k < K) ? W[k * N + n] : (uint16_t)0;
    }
}

hipError_t launch_gather_wo(const void* W, int64_t K, int64_t N, const int32_t* O, int64_t nO, int64_t P, void* WO,
                            hipStream_t stream) {
    if (N == 0 || P == 0) return hipSuccess;
    dim3 g((unsigned)ceil_div(N, 256), (unsigned)(P < 65535 ? P : 65535));
    gather_wo_kernel<<<g, 256, 0, stream>>>((const uint16_t*)W, K, N, O, nO, P, (uint16_t*)WO);
    return hipGetLastError();
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    const int64_t blocks = ceil_div(n, 256);
    fill_zero_kernel<<<(unsigned)(blocks < 65536 ? blocks : 65536), 256, 0, stream>>>(p, n);
    return hipGetLastError();
}

int64_t weight_splits(int64_t K) {
    int64_t s = ceil_div(K, 256);
    return s < 1 ? 1 : (s > 64 ? 64 : s);
}

hipError_t launch_weight(int dt, const void* W, int64_t K, int64_t N, int8_t* Wq, float* w_scale,
                         const uint32_t* skip, hipStream_t stream) {
    if (N == 0) return hipSuccess;
    hipError_t e = launch_fill_zero(w_scale, N, stream);
    if (e != hipSuccess || K == 0) return e;
    const int64_t S = weight_splits(K);
    const int64_t rps = ceil_div(K, S);
    dim3 g1((unsigned)ceil_div(N, 512), (unsigned)ceil_div(K, rps));
    dim3 g2((unsigned)ceil_div(N, 64), (unsigned)ceil_div(K, 128));
    if (dt == F16) {
        colmax_kernel<F16><<<g1, 256, 0, stream>>>((const uint16_t*)W, K, N, rps, skip, w_scale);
        quantize_weight_kernel<F16><<<g2, 256, 0, stream>>>((const uint16_t*)W, K, N, w_scale, 1, K, skip, Wq);
    } else {
        colmax_kernel<BF16><<<g1, 256, 0, stream>>>((const uint16_t*)W, K, N, rps, skip, w_scale);
        quantize_weight_kernel<BF16><<<g2, 256, 0, stream>>>((const uint16_t*)W, K, N, w_scale, 1, K, skip, Wq);
    }
    return hipGetLastError();
}

hipError_t launch_quantize_weight_groups(int dt, const void* W, int64_t K, int64_t N, const float* s_w, int64_t G,
                                         int8_t* Wq, hipStream_t stream) {
    if (N == 0 || K == 0) return hipSuccess;
    dim3 g2((unsigned)ceil_div(N, 64), (unsigned)ceil_div(K, 128));
    if (dt == F16)
        quantize_weight_kernel<F16><<<g2, 256, 0, stream>>>((const uint16_t*)W, K, N, s_w, K / G, G, nullptr, Wq);
    else
        quantize_weight_kernel<BF16><<<g2, 256, 0, stream>>>((const uint16_t*)W, K, N, s_w, K / G, G, nullptr, Wq);
    return hipGetLastError();
}

}  // namespace llmint8
