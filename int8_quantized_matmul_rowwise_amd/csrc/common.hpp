// Device-side helpers shared by the llmint8 kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace llmint8 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

enum Dtype : int { F16 = 0, BF16 = 1 };

constexpr int kWave = 64;

// 16-bit pattern -> fp32, exact.
template <int DT>
__device__ __forceinline__ float to_f32(uint16_t h) {
    if constexpr (DT == F16) {
        return (float)__builtin_bit_cast(_Float16, h);
    } else {
        return __builtin_bit_cast(float, (uint32_t)h << 16);
    }
}

// fp32 -> 16-bit pattern, round to nearest even (hardware conversion in both cases).
template <int DT>
__device__ __forceinline__ uint16_t from_f32(float f) {
    if constexpr (DT == F16) {
        return __builtin_bit_cast(uint16_t, (_Float16)f);
    } else {
        return __builtin_bit_cast(uint16_t, (__bf16)f);
    }
}

// The vector-wise code: inv = s > 0 ? RN32(127/s) : 0 (IEEE division, correctly
// rounded under the default HIP float settings), q = clamp(rne(RN32(x*inv)), -127, 127).
__device__ __forceinline__ float inv_scale(float s) { return s > 0.0f ? 127.0f / s : 0.0f; }

__device__ __forceinline__ int quantize(float x, float inv) {
    float v = __builtin_rintf(__fmul_rn(x, inv));
    v = v > 127.0f ? 127.0f : v;
    v = v < -127.0f ? -127.0f : v;
    return (int)v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
    return v;
}

__host__ __device__ constexpr int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }
__host__ __device__ constexpr int64_t ceil_div(int64_t v, int64_t m) { return (v + m - 1) / m; }

// Small batches also keep Xq in the small-batch product kernel's operand layout: blocks of
// 16 rows x 64 columns (1 KB, row-major inside), the nsteps = ceil(K/64) blocks of one
// group of 16 rows in K order, then the next group.  One operand load of that kernel (16
// rows x 64 bytes) is then one 1 KB block, eight whole cache lines, instead of 16 halves
// of lines.  Columns K..64*nsteps of a block are 0; rows past M are not stored.
__host__ __device__ constexpr int64_t xqb_offset(int64_t r, int64_t k, int64_t nsteps) {
    return ((r >> 4) * nsteps + (k >> 6)) * 1024 + (r & 15) * 64 + (k & 63);
}

}  // namespace llmint8
