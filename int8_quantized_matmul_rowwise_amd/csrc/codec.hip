// Block-wise absmax int8 codec of a flat fp32 tensor ("llama3-model-quantization" talk
// summary, Key Points, 8-bit optimizers: the state is cut into blocks, each block is
// normalised by its own maximum and kept as 8-bit values).  The linear code, with the same
// quantizer as the matmul:
//   absmax[b] = max |x| over block b = elements [b*block, min((b+1)*block, n)),
//   q = clamp(rne(RN32(x * RN32(127 / absmax[b]))), -127, 127)   (absmax 0: q = 0),
//   decode x' = RN32((float)q * RN32(absmax[b] / 127)).
// HBM-bound: 4 + 1 bytes per element to code, 1 + 4 to decode (+ 4 per block).  One wave
// takes one block (blocks of 256 elements and more) or one segment of SEG lanes takes one
// block (64, 128), each lane 4 consecutive elements per 16-byte access, so that a wave's
// access is 1 KB contiguous; the workgroups walk the blocks grid-stride.
#include "common.hpp"
#include "launch.hpp"

namespace llmint8 {

namespace {

// The 4 codes of 4 elements, one per byte (the low byte of RN32(clamp(v) + 1.5 * 2^23) is
// rne(v) in two's complement: the sum lies in [2^23, 2^24), where the float spacing is 1).
__device__ __forceinline__ uint32_t code4(const float (&e)[4], float inv) {
    uint32_t t[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float v = __fmul_rn(e[j], inv);
        v = fminf(fmaxf(v, -127.0f), 127.0f);
        t[j] = __builtin_bit_cast(uint32_t, __fadd_rn(v, 12582912.0f));
    }
    return __builtin_amdgcn_perm(t[1], t[0], 0x0c0c0400u) | __builtin_amdgcn_perm(t[3], t[2], 0x04000c0cu);
}

// NV: 16-byte groups per lane; SEG: lanes per block (64, or 16 / 32 for blocks of 64 / 128).
template <int NV, int SEG>
__global__ __launch_bounds__(256) void block_quantize_kernel(const float* __restrict__ x, int64_t n, int64_t block,
                                                             int64_t nblocks, int8_t* __restrict__ q,
                                                             float* __restrict__ absmax) {
    constexpr int BPW = 64 / SEG;  // blocks per wave pass
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int sub = lane / SEG, sl = lane % SEG;
    const int64_t nwaves = (int64_t)gridDim.x * 4;
    for (int64_t b0 = ((int64_t)blockIdx.x * 4 + w) * BPW; b0 < nblocks; b0 += nwaves * BPW) {
        const int64_t b = b0 + sub;
        const int64_t lo = b * block;
        float e[NV][4];
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int64_t i = lo + 4 * ((int64_t)j * SEG + sl);
            if (b < nblocks && i + 4 <= n) {
                const v4f t = *(const v4f*)(x + i);
#pragma unroll
                for (int k = 0; k < 4; ++k) e[j][k] = t[k];
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k) e[j][k] = (b < nblocks && i + k < n) ? x[i + k] : 0.0f;
            }
        }
        float m = 0.0f;
#pragma unroll
        for (int j = 0; j < NV; ++j)
#pragma unroll
            for (int k = 0; k < 4; ++k) m = fmaxf(m, __builtin_fabsf(e[j][k]));
#pragma unroll
        for (int off = SEG / 2; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
        const float inv = inv_scale(m);
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int64_t i = lo + 4 * ((int64_t)j * SEG + sl);
            const uint32_t c = code4(e[j], inv);
            if (b < nblocks && i + 4 <= n) {
                *(uint32_t*)(q + i) = c;
            } else if (b < nblocks) {
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    if (i + k < n) q[i + k] = (int8_t)(c >> (8 * k));
            }
        }
        if (sl == 0 && b < nblocks) absmax[b] = m;
    }
}

template <int NV, int SEG>
__global__ __launch_bounds__(256) void block_dequantize_kernel(const int8_t* __restrict__ q,
                                                               const float* __restrict__ absmax, int64_t n,
                                                               int64_t block, int64_t nblocks,
                                                               float* __restrict__ x) {
    constexpr int BPW = 64 / SEG;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int sub = lane / SEG, sl = lane % SEG;
    const int64_t nwaves = (int64_t)gridDim.x * 4;
    for (int64_t b0 = ((int64_t)blockIdx.x * 4 + w) * BPW; b0 < nblocks; b0 += nwaves * BPW) {
        const int64_t b = b0 + sub;
        if (b >= nblocks) continue;
        const int64_t lo = b * block;
        const float step = absmax[b] / 127.0f;
        uint32_t c[NV];
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int64_t i = lo + 4 * ((int64_t)j * SEG + sl);
            if (i + 4 <= n) {
                c[j] = *(const uint32_t*)(q + i);
            } else {
                c[j] = 0u;
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    if (i + k < n) c[j] |= (uint32_t)(uint8_t)q[i + k] << (8 * k);
            }
        }
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int64_t i = lo + 4 * ((int64_t)j * SEG + sl);
            v4f t;
#pragma unroll
            for (int k = 0; k < 4; ++k) t[k] = __fmul_rn((float)(int8_t)(c[j] >> (8 * k)), step);
            if (i + 4 <= n) {
                *(v4f*)(x + i) = t;
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    if (i + k < n) x[i + k] = t[k];
            }
        }
    }
}

// Workgroups: enough for every block, at most 8 per CU (the loop strides over the rest).
unsigned codec_grid(int64_t nblocks, int blocks_per_wave) {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus = 256;
    const int64_t need = ceil_div(nblocks, 4 * (int64_t)blocks_per_wave);
    const int64_t cap = (int64_t)cus * 8;
    return (unsigned)(need < cap ? need : cap);
}

template <bool QUANT, int NV, int SEG>
hipError_t codec_launch(const float* x, const int8_t* qin, const float* amin, int64_t n, int64_t block, int8_t* qout,
                        float* amout, float* xout, hipStream_t stream) {
    const int64_t nblocks = ceil_div(n, block);
    const unsigned grid = codec_grid(nblocks, 64 / SEG);
    if (QUANT)
        block_quantize_kernel<NV, SEG><<<grid, 256, 0, stream>>>(x, n, block, nblocks, qout, amout);
    else
        block_dequantize_kernel<NV, SEG><<<grid, 256, 0, stream>>>(qin, amin, n, block, nblocks, xout);
    return hipGetLastError();
}

template <bool QUANT>
hipError_t codec_dispatch(const float* x, const int8_t* qin, const float* amin, int64_t n, int64_t block,
                          int8_t* qout, float* amout, float* xout, hipStream_t stream) {
    switch (block) {
        case 64: return codec_launch<QUANT, 1, 16>(x, qin, amin, n, block, qout, amout, xout, stream);
        case 128: return codec_launch<QUANT, 1, 32>(x, qin, amin, n, block, qout, amout, xout, stream);
        case 256: return codec_launch<QUANT, 1, 64>(x, qin, amin, n, block, qout, amout, xout, stream);
        case 512: return codec_launch<QUANT, 2, 64>(x, qin, amin, n, block, qout, amout, xout, stream);
        case 1024: return codec_launch<QUANT, 4, 64>(x, qin, amin, n, block, qout, amout, xout, stream);
        case 2048: return codec_launch<QUANT, 8, 64>(x, qin, amin, n, block, qout, amout, xout, stream);
        default: return codec_launch<QUANT, 16, 64>(x, qin, amin, n, block, qout, amout, xout, stream);
    }
}

}  // namespace

bool codec_block_ok(int64_t block) { return block >= 64 && block <= 4096 && (block & (block - 1)) == 0; }

hipError_t launch_block_quantize(const float* x, int64_t n, int64_t block, int8_t* q, float* absmax,
                                 hipStream_t stream) {
    if (n == 0) return hipSuccess;
    return codec_dispatch<true>(x, nullptr, nullptr, n, block, q, absmax, nullptr, stream);
}

hipError_t launch_block_dequantize(const int8_t* q, const float* absmax, int64_t n, int64_t block, float* x,
                                   hipStream_t stream) {
    if (n == 0) return hipSuccess;
    return codec_dispatch<false>(nullptr, q, absmax, n, block, nullptr, nullptr, x, stream);
}

}  // namespace llmint8
