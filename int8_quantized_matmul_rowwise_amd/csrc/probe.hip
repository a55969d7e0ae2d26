// Measurement probes for the benchmark (libllmint8_probe.so; not part of libllmint8.so and
// not on the matmul's path): the part's sustained int8 MFMA rate and shader clock, and its
// HBM stream-read rate, measured on the box the benchmark runs on.
#include <hip/hip_runtime.h>
#include <stdint.h>

#define PROBE_API extern "C" __attribute__((visibility("default")))

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;  // two per SIMD, like the product kernel

// splitmix-style hash of a lane's position: operand bytes that look random
__device__ uint32_t mix(uint32_t x) {
    x ^= x >> 16;
    x *= 0x7feb352dU;
    x ^= x >> 15;
    x *= 0x846ca68bU;
    x ^= x >> 16;
    return x;
}

// Every wave runs `iters` rounds of 8 independent 32x32x32 int8 MFMAs from registers (no
// memory traffic).  mode 0: zero operands.  mode 1: two sets of random operands, alternated
// from one MFMA to the next, so the matrix unit's inputs change as they do in a product
// that streams its operands.  Thread 0 of each workgroup records the shader clock counter
// (s_memtime) and the 100 MHz real-time counter (s_memrealtime) around the loop.
__global__ __launch_bounds__(64 * kWaves) void mfma_i8_probe(int64_t iters, int mode, int32_t* out, uint64_t* clk) {
    __shared__ int8_t hold[96 * 1024];  // one workgroup per compute unit
    const int tid = threadIdx.x;
    const uint32_t seed = (blockIdx.x * 64 * kWaves + tid) * 16u;
    v4i a[2], b[2];
    for (int s = 0; s < 2; ++s)
        for (int e = 0; e < 4; ++e) {
            a[s][e] = mode ? (int)mix(seed + 4 * s + e) : 0;
            b[s][e] = mode ? (int)mix(seed + 8 + 4 * s + e) : 0;
        }
    if (tid == 0) hold[0] = (int8_t)mode;
    v16i acc[8];
    for (int j = 0; j < 8; ++j) acc[j] = v16i{};
    __syncthreads();
    const uint64_t t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[j & 1], b[(j >> 1) & 1], acc[j], 0, 0, 0);
    }
    const uint64_t t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    int32_t s = 0;
    for (int j = 0; j < 8; ++j)
        for (int e = 0; e < 16; ++e) s += acc[j][e];
    out[blockIdx.x * 64 * kWaves + tid] = s + hold[0];
    if (tid == 0) {
        clk[4 * blockIdx.x + 0] = t0;
        clk[4 * blockIdx.x + 1] = t1;
        clk[4 * blockIdx.x + 2] = r0;
        clk[4 * blockIdx.x + 3] = r1;
    }
}

// Sum of a buffer's 32-bit words: 16-byte loads per lane, grid-stride, one partial per
// thread (the read itself is what is timed).
__global__ __launch_bounds__(256) void stream_read_probe(const u32x4* p, int64_t n16, uint32_t* out) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    uint32_t s = 0;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 v0 = p[i], v1 = p[i + stride], v2 = p[i + 2 * stride], v3 = p[i + 3 * stride];
        s += v0.x ^ v0.y ^ v0.z ^ v0.w ^ v1.x ^ v1.y ^ v1.z ^ v1.w ^ v2.x ^ v2.y ^ v2.z ^ v2.w ^ v3.x ^ v3.y ^ v3.z ^ v3.w;
    }
    for (; i < n16; i += stride) {
        const u32x4 v = p[i];
        s += v.x ^ v.y ^ v.z ^ v.w;
    }
    out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

// grid: workgroups (one per compute unit: pass the CU count); out: grid * 512 int32;
// clk: grid * 4 uint64.  Returns the launch status (0 = hipSuccess).
PROBE_API int llmint8_probe_mfma_i8(int grid, int64_t iters, int mode, int32_t* out, uint64_t* clk, void* stream) {
    if (grid <= 0 || iters <= 0 || !out || !clk) return (int)hipErrorInvalidValue;
    mfma_i8_probe<<<grid, 64 * kWaves, 0, (hipStream_t)stream>>>(iters, mode, out, clk);
    return (int)hipGetLastError();
}

// p: bytes (a multiple of 16, 16-byte aligned); out: grid * 256 uint32.
PROBE_API int llmint8_probe_stream_read(const void* p, int64_t bytes, int grid, uint32_t* out, void* stream) {
    if (!p || bytes <= 0 || bytes % 16 || grid <= 0 || !out) return (int)hipErrorInvalidValue;
    stream_read_probe<<<grid, 256, 0, (hipStream_t)stream>>>((const u32x4*)p, bytes / 16, out);
    return (int)hipGetLastError();
}
