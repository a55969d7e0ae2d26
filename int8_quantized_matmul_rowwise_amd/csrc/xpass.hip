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
// rows of X in flight per thread of the detection (16 x 16 B: with three to six
// workgroups per compute unit, enough bytes in flight to stream X at HBM rate)
constexpr int kDetectRows = 16;

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
        for (; r + 4 * (kDetectRows - 1) < r1; r += 4 * kDetectRows) {  // kDetectRows rows in flight per thread
            u32x4 v[kDetectRows];
#pragma unroll
            for (int u = 0; u < kDetectRows; ++u) v[u] = *(const u32x4*)(col + (r + 4 * u) * K);
#pragma unroll
            for (int u = 0; u < kDetectRows; ++u)
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
                                                       int32_t* __restrict__ n_out, int32_t* __restrict__ zero,
                                                       int64_t n_zero) {
    __shared__ uint32_t bits[kMaxKw];
    __shared__ int32_t wsum[16];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    for (int64_t i = tid; i < n_zero; i += 1024) zero[i] = 0;
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

// Bitmap of a caller's list of outlier columns (fixed-outlier path), one workgroup:
// bits in LDS (atomicOr), then the words out.  Entries outside [0, K) are ignored.
__global__ __launch_bounds__(1024) void list_bitmap_kernel(int64_t K, const int32_t* __restrict__ O, int64_t nO,
                                                           uint32_t* __restrict__ partial) {
    __shared__ uint32_t bits[kMaxKw];
    const int tid = threadIdx.x;
    const int64_t Kw = ceil_div(K, 32);
    for (int64_t w = tid; w < Kw; w += 1024) bits[w] = 0;
    __syncthreads();
    for (int64_t t = tid; t < nO; t += 1024) {
        const int64_t k = O[t];
        if (k >= 0 && k < K) atomicOr(&bits[k >> 5], 1u << (k & 31));
    }
    __syncthreads();
    for (int64_t w = tid; w < Kw; w += 1024) partial[w] = bits[w];
}

hipError_t launch_list_bitmap(int64_t K, const int32_t* O, int64_t nO, uint32_t* partial, hipStream_t stream) {
    if (K == 0) return hipSuccess;
    list_bitmap_kernel<<<1, 1024, 0, stream>>>(K, O, nO, partial);
    return hipGetLastError();
}

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
                          int32_t* n_out, hipStream_t stream, int32_t* zero, int64_t n_zero) {
    const int64_t nrb = detect_row_blocks(M);
    const int64_t Kw = (M > 0 && K > 0) ? ceil_div(K, 32) : 0;
    compact_kernel<<<1, 1024, 0, stream>>>(partial, nrb, Kw, bitmap, O, n_out, zero, zero ? n_zero : 0);
    return hipGetLastError();
}

}  // namespace llmint8

// ---------------------------------------------------------------------------
// Row coding of the tiled path (after detect and compact), and the small-batch X pass
// (M <= kSmallM rows, K <= kSmallK): one workgroup for at most 64 KB of X, else two
// launches over 512-column slabs.
namespace llmint8 {


// ---- per-chunk arithmetic of the row coding (a chunk: 8 consecutive 16-bit elements in
// four dwords; o: its 8 outlier bits; any: some lane of the wave has o != 0, wave-uniform)
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// 0xffff over the halves of dword d (elements 2d, 2d+1) whose outlier bits are set
__device__ __forceinline__ uint32_t outlier_halves(uint32_t o, int d) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_sbfe((int)o, 2 * d, 1);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_sbfe((int)o, 2 * d + 1, 1);
    return (lo & 0xffffu) | (hi & 0xffff0000u);
}

// 0xff over the bytes whose bit is set in the low 4 bits of b (no carries: the four
// shifted copies of b do not overlap)
__device__ __forceinline__ uint32_t byte_mask4(uint32_t b) { return ((b * 0x00204081u) & 0x01010101u) * 0xffu; }

// Running max of the magnitudes of the non-outlier elements.  For finite fp16 and bf16
// values the order of |x| is the unsigned order of the pattern without its sign bit, so the
// max is taken on those 15-bit integers, two per instruction.
__device__ __forceinline__ u16x2 absmax_bits(u16x2 acc, const u32x4& x, uint32_t o, bool any) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        uint32_t a = x[d] & 0x7fff7fffu;
        if (any) a &= ~outlier_halves(o, d);
        acc = __builtin_elementwise_max(acc, __builtin_bit_cast(u16x2, a));
    }
    return acc;
}

// Codes of a chunk, byte j of dword d for element 4d + j: clamp(rne(RN32(x * inv)), -127,
// 127), 0 in outlier columns.  Rounding to an integer by adding 1.5 * 2^23: the sum lies
// in [2^23, 2^24), where the float spacing is 1, so the add rounds to nearest even and the
// integer sits in the low mantissa bits (its low byte is the two's-complement code).  The
// clamp is never taken here: inv = RN32(127/s) with s the largest |x| of the row's
// non-outlier columns, so for them |RN32(x * inv)| <= RN32(s * inv) < 127.5 and the code is
// within +-127 as it is; the outlier columns' bytes (any value, even past the add's range)
// are masked to 0 below.
template <int DT>
__device__ __forceinline__ u32x2 code_chunk(const u32x4& x, uint32_t o, float inv, bool any) {
    uint32_t t[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float f = to_f32<DT>((uint16_t)(x[j >> 1] >> (16 * (j & 1))));
        t[j] = __builtin_bit_cast(uint32_t, __fadd_rn(__fmul_rn(f, inv), 12582912.0f));
    }
    u32x2 q;
    q[0] = __builtin_amdgcn_perm(t[1], t[0], 0x0c0c0400u) | __builtin_amdgcn_perm(t[3], t[2], 0x04000c0cu);
    q[1] = __builtin_amdgcn_perm(t[5], t[4], 0x0c0c0400u) | __builtin_amdgcn_perm(t[7], t[6], 0x04000c0cu);
    if (any) {
        q[0] &= ~byte_mask4(o & 0xfu);
        q[1] &= ~byte_mask4(o >> 4);
    }
    return q;
}

// The set-up shared by the row coding and the W_O gather (a block of 256 threads): the
// bitmap's Kw words in bits[] and, per word, the number of outlier columns before it in
// wrank[] (both LDS; a block-wide scan of popcounts).  Returns the number of outlier
// columns.
__device__ __forceinline__ int32_t bitmap_ranks(const uint32_t* __restrict__ bitmap, int64_t Kw, uint32_t* bits,
                                                int32_t* wrank, int32_t* wsum) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    for (int64_t w = tid; w < Kw; w += 256) bits[w] = bitmap[w];
    __syncthreads();
    // thread tid takes words [tid*wpt, (tid+1)*wpt); its first rank is the exclusive prefix
    // of the popcounts before them
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
    for (int64_t w = tid * wpt; w < (tid + 1) * wpt && w < Kw; ++w) {
        wrank[w] = pos;
        pos += __popc(bits[w]);
    }
    __syncthreads();
    return total;
}

// The column of outlier rank t < total from that set-up: the last word whose rank is at
// most t holds it (empty words after it have larger ranks), as its (t - rank)-th set bit.
__device__ __forceinline__ int64_t outlier_column(int32_t t, int64_t Kw, const uint32_t* bits, const int32_t* wrank) {
    int64_t lo = 0, hi = Kw - 1;
    while (lo < hi) {
        const int64_t mid = (lo + hi + 1) >> 1;
        if (wrank[mid] <= t) lo = mid;
        else hi = mid - 1;
    }
    uint32_t b = bits[lo];
    for (int32_t k = t - wrank[lo]; k > 0; --k) b &= b - 1;
    return 32 * lo + __ffs(b) - 1;
}

// WO[n,t] = (dtype) Wq[n, O[t]] (exact; zero up to the next multiple of 32) for the 64 rows
// of Wq from n0, with O[t] = col_of(t) for t < nO: thread: column t0 + tid%32 of W_O, rows
// tid/32 + 8k; one column lookup, 8 independent Wq loads.
template <int DT, class ColOf>
__device__ __forceinline__ void gather_wo_rows(int64_t n0, int64_t K, int32_t nO, ColOf col_of,
                                               const int8_t* __restrict__ Wq, int64_t N, uint16_t* __restrict__ WO,
                                               int64_t xo_pitch) {
    const int tid = threadIdx.x;
    const int32_t P = (nO + 31) & ~31;
    const int rr = tid >> 5;
    for (int32_t t0 = 0; t0 < P; t0 += 32) {
        const int32_t t = t0 + (tid & 31);
        const int64_t col = t < nO ? col_of(t) : -1;
        uint16_t v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int64_t n = n0 + rr + 8 * k;
            v[k] = (col >= 0 && n < N) ? from_f32<DT>((float)Wq[n * K + col]) : (uint16_t)0;
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int64_t n = n0 + rr + 8 * k;
            if (n < N) WO[n * xo_pitch + t] = v[k];
        }
    }
}

// Code the rows.  The first n_wo workgroups gather W_O (gather_wo_rows), 64 rows of Wq
// each, from the O written by the compaction; they come first so that their scattered
// loads overlap the row work instead of trailing it.  The other `groups` workgroups each
// take rows g, g + groups, ...: for
// row i, s_x[i] = max over the non-outlier columns of |X[i,j]|; Xq[i,j] = 0 for j in O,
// else the vector-wise code; Xq[i, K..pitch) = 0; XO[i,t] = X[i, O[t]] for t < n_O, 0 up
// to the next multiple of 32.  Set-up once per workgroup: the bitmap in LDS and, per
// word, the number of outlier columns before it (a block-wide scan of popcounts), which
// gives the rank t of every outlier column.  HOLD > 0: a row stays in registers (HOLD
// 16-byte chunks per thread, K <= 2048 * HOLD) between its max and its coding, else each
// row is read twice.  (A second register set, to load the next row while one is coded,
// costs more in occupancy than it gains.)
template <int DT, int HOLD>
__global__ __launch_bounds__(256) void code_rows_kernel(const uint16_t* __restrict__ X, int64_t M, int64_t K,
                                                        const uint32_t* __restrict__ bitmap, int32_t* __restrict__ O,
                                                        int32_t* __restrict__ n_out, int8_t* __restrict__ Xq,
                                                        int64_t xq_pitch, float* __restrict__ s_x,
                                                        uint16_t* __restrict__ XO, int64_t xo_pitch,
                                                        const int8_t* __restrict__ Wq, int64_t N,
                                                        uint16_t* __restrict__ WO, int64_t n_wo, int64_t groups) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    if ((int64_t)blockIdx.x < n_wo) {
        gather_wo_rows<DT>((int64_t)blockIdx.x * 64, K, *n_out, [&](int32_t t) { return (int64_t)O[t]; }, Wq, N, WO,
                           xo_pitch);
        return;
    }
    // dynamic LDS, sized to K: the bitmap, then the outlier count before each word
    extern __shared__ uint32_t dyn_lds[];
    __shared__ float red[2][4];
    __shared__ int32_t wsum[4];
    const int64_t g = (int64_t)blockIdx.x - n_wo;
    const int64_t nch = K / 8, Kw = ceil_div(K, 32);
    uint32_t* bits = dyn_lds;
    int32_t* wrank = (int32_t*)(dyn_lds + Kw);
    constexpr int H = HOLD > 0 ? HOLD : 1;
    u32x4 va[H];
    // through a buffer resource over the row: 32-bit lane offsets (the whole offset, which
    // the range check covers), no 64-bit address per chunk, and chunks past the row read 0,
    // so every load is issued
    auto load_row = [&](u32x4(&v)[H], int64_t i) {
        const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc((void*)(X + i * K), (short)0, (int)(2 * K),
                                                                            0x00020000);
        uint32_t off = 16 * tid;  // stepped behind an opaque copy: one register, not one per chunk
#pragma unroll
        for (int h = 0; h < H; ++h) {
            v[h] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rr, off, 0, 0));
            off += 16 * 256;
            asm volatile("" : "+v"(off));
        }
    };
    if constexpr (HOLD > 0) load_row(va, g);  // in flight during the set-up

    const int32_t total = bitmap_ranks(bitmap, Kw, bits, wrank, wsum);
    const int32_t P = (total + 31) & ~31;

    auto obits = [&](int64_t c) { return (bits[c >> 2] >> (8 * (c & 3))) & 0xffu; };
    auto wave_any = [](uint32_t o) { return __builtin_amdgcn_ballot_w64(o != 0u) != 0; };

    // one row: its max, its codes, its outlier values (from the chunk in hand, at their
    // ranks), its padding.  par: which slot of red this row uses (a slot is written again
    // only two rows later, after a barrier every wave has passed, so one barrier per row).
    auto process = [&](const u32x4(&v)[H], int64_t i, int par) {
        const uint16_t* row = X + i * K;
        u16x2 mb = {0, 0};
        if constexpr (HOLD > 0) {
#pragma unroll
            for (int h = 0; h < HOLD; ++h) {
                const int c = tid + 256 * h;
                const uint32_t o = c < nch ? obits(c) : 0u;  // chunks past the row hold zeros
                mb = absmax_bits(mb, v[h], o, wave_any(o));
            }
        } else {
            for (int64_t c = tid; c < nch; c += 256) {
                const uint32_t o = obits(c);
                mb = absmax_bits(mb, *(const u32x4*)(row + c * 8), o, wave_any(o));
            }
        }
        float m = to_f32<DT>(mb[0] > mb[1] ? mb[0] : mb[1]);
        m = wave_max(m);
        if (lane == 0) red[par][wv] = m;
        __syncthreads();
        const float s = fmaxf(fmaxf(red[par][0], red[par][1]), fmaxf(red[par][2], red[par][3]));
        const float inv = inv_scale(s);
        int8_t* qrow = Xq + i * xq_pitch;
        uint16_t* xo = XO + i * xo_pitch;
        auto code_store = [&](const u32x4& x, int64_t c) {
            const uint32_t o = obits(c);
            const bool any = wave_any(o);
            *(u32x2*)(qrow + c * 8) = code_chunk<DT>(x, o, inv, any);
            if (any && o) {
                int32_t r = wrank[c >> 2] + __popc(bits[c >> 2] & ((1u << (8 * (c & 3))) - 1u));
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    if ((o >> j) & 1u) xo[r++] = (uint16_t)(x[j >> 1] >> (16 * (j & 1)));
                }
            }
        };
        if constexpr (HOLD > 0) {
            // one chunk at a time: the index is opaque per chunk (and memory is clobbered), so
            // the compiler neither keeps the first pass's flags nor codes several chunks ahead
            int tx = tid;
#pragma unroll
            for (int h = 0; h < HOLD; ++h) {
                asm volatile("" : "+v"(tx)::"memory");
                const int c = tx + 256 * h;
                if (c < nch) code_store(v[h], c);
            }
        } else {
            for (int64_t c = tid; c < nch; c += 256) code_store(*(const u32x4*)(row + c * 8), c);
        }
        for (int64_t c = nch + tid; c < xq_pitch / 8; c += 256) *(u32x2*)(qrow + c * 8) = u32x2{0u, 0u};
        for (int64_t t = total + tid; t < P; t += 256) xo[t] = 0;
        if (tid == 0) s_x[i] = s;
    };

    int par = 0;
    for (int64_t i = g; i < M; i += groups, par ^= 1) {
        if (HOLD > 0 && i != g) load_row(va, i);
        process(va, i, par);
    }
}

// The whole small-batch X pass in one workgroup, for M * K <= kOneMaxElems (64 KB of X:
// one compute unit keeps too few loads in flight for more -- 256 KB took 30 us this way,
// against 9 us for the two launches): X is read once, into registers (up to kOneChunks
// 8-column chunks per thread, chunk i of the
// row-major X at X + 8 i), and every later step works on them and on LDS: detection (the
// chunks' outlier bits ORed into an LDS bitmap), the list O and the per-word ranks (a
// block scan of the words' popcounts, one word per thread: K <= 32768), the row maxima
// over the non-outlier columns (per row in LDS, one atomic per wave when the wave's 64
// chunks lie in one row) and the coding (also into the blocked copy Xqb when it is not
// NULL).  The same per-chunk arithmetic as the two-launch
// path, so the results are the same bits.  All indices fit 32 bits (M * K <= 32768).
constexpr int kOneChunks = 4;
constexpr int64_t kOneMaxElems = 1024 * kOneChunks * 8;

template <int DT>
__global__ __launch_bounds__(1024) void xpass_one_kernel(const uint16_t* __restrict__ X, int M, int K, float tau,
                                                         uint32_t* __restrict__ bitmap, int32_t* __restrict__ O,
                                                         int32_t* __restrict__ n_out, int8_t* __restrict__ Xq,
                                                         int xq_pitch, int8_t* __restrict__ Xqb, int nsteps,
                                                         float* __restrict__ s_x, uint16_t* __restrict__ XO,
                                                         int xo_pitch) {
    __shared__ uint32_t bits[1024];
    __shared__ int32_t wrank[1024];
    __shared__ uint32_t rmax[kSmallM];
    __shared__ int32_t wsum[16];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int C = K / 8, items = M * C, Kw = (K + 31) / 32;
    // chunk tid + 1024 u is row r[u], chunk c[u] of it (stepped without divisions)
    int r[kOneChunks], c[kOneChunks];
    {
        const int q = 1024 / C, rm = 1024 % C;
        int rr = tid / C, cc = tid % C;
#pragma unroll
        for (int u = 0; u < kOneChunks; ++u) {
            r[u] = rr;
            c[u] = cc;
            rr += q;
            cc += rm;
            if (cc >= C) {
                cc -= C;
                ++rr;
            }
        }
    }
    u32x4 v[kOneChunks];
#pragma unroll
    for (int u = 0; u < kOneChunks; ++u) {
        const int i = tid + 1024 * u;
        v[u] = i < items ? *(const u32x4*)(X + 8 * i) : u32x4{0u, 0u, 0u, 0u};
    }
    bits[tid] = 0;
    if (tid < kSmallM) rmax[tid] = 0;
    __syncthreads();
    // detection: |x| > tau, compared in fp32
#pragma unroll
    for (int u = 0; u < kOneChunks; ++u) {
        if (tid + 1024 * u >= items) continue;
        uint32_t mask = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            mask |= (__builtin_fabsf(to_f32<DT>((uint16_t)(v[u][j >> 1] >> (16 * (j & 1))))) > tau ? 1u : 0u) << j;
        if (mask) atomicOr(&bits[c[u] >> 2], mask << (8 * (c[u] & 3)));
    }
    __syncthreads();
    // O in ascending column order, n_O, and each word's rank of its first outlier column
    const uint32_t word = tid < Kw ? bits[tid] : 0u;
    const int32_t cnt = __popc(word);
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
    for (int q = 0; q < 16; ++q) {
        pos += q < wv ? wsum[q] : 0;
        total += wsum[q];
    }
    if (tid < Kw) {
        wrank[tid] = pos;
        bitmap[tid] = word;
        for (uint32_t wd = word, t = (uint32_t)pos; wd; wd &= wd - 1) O[t++] = 32 * tid + __ffs(wd) - 1;
    }
    if (tid == 0) *n_out = total;
    auto obits = [&](int cc) { return (bits[cc >> 2] >> (8 * (cc & 3))) & 0xffu; };
    // row maxima of the magnitudes (15-bit patterns) over the non-outlier columns
#pragma unroll
    for (int u = 0; u < kOneChunks; ++u) {
        if (1024 * u + 64 * wv >= items) continue;  // the wave's first chunk (wave-uniform)
        const bool valid = tid + 1024 * u < items;
        uint32_t m = 0;
        if (valid) {
            const u16x2 mb = absmax_bits(u16x2{0, 0}, v[u], obits(c[u]), true);
            m = mb[0] > mb[1] ? mb[0] : mb[1];
        }
        // the wave's 64 chunks in one row: reduce in the wave (patterns below 2^15 are exact
        // floats); chunks past the end have rows >= M, so a partial wave takes the other way
        const int r0 = __builtin_amdgcn_readfirstlane(r[u]);
        if (r0 == __shfl(r[u], 63, kWave)) {
            m = (uint32_t)wave_max((float)m);
            if (lane == 0) atomicMax(&rmax[r0], m);
        } else if (valid) {
            atomicMax(&rmax[r[u]], m);
        }
    }
    __syncthreads();
    // codes, outlier values at their ranks, scales and padding
#pragma unroll
    for (int u = 0; u < kOneChunks; ++u) {
        if (tid + 1024 * u >= items) continue;
        const int rr = r[u], cc = c[u];
        const float inv = inv_scale(to_f32<DT>((uint16_t)rmax[rr]));
        const uint32_t o = obits(cc);
        const u32x2 q = code_chunk<DT>(v[u], o, inv, true);
        *(u32x2*)(Xq + rr * xq_pitch + 8 * cc) = q;
        if (Xqb) *(u32x2*)(Xqb + xqb_offset(rr, 8 * cc, nsteps)) = q;
        if (o) {
            int32_t t = wrank[cc >> 2] + __popc(bits[cc >> 2] & ((1u << (8 * (cc & 3))) - 1u));
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if ((o >> j) & 1u) XO[rr * xo_pitch + t++] = (uint16_t)(v[u][j >> 1] >> (16 * (j & 1)));
        }
    }
    if (tid < M) s_x[tid] = to_f32<DT>((uint16_t)rmax[tid]);
    const int pad_c = (xq_pitch - K) / 8, pad_o = ((total + 31) & ~31) - total;
    for (int e = tid; e < M * pad_c; e += 1024)
        *(u32x2*)(Xq + (e / pad_c) * xq_pitch + K + 8 * (e % pad_c)) = u32x2{0u, 0u};
    const int pad_b = 8 * nsteps - K / 8;  // the blocked copy's zero columns, K .. 64 nsteps
    if (Xqb)
        for (int e = tid; e < M * pad_b; e += 1024)
            *(u32x2*)(Xqb + xqb_offset(e / pad_b, K + 8 * (e % pad_b), nsteps)) = u32x2{0u, 0u};
    for (int e = tid; e < M * pad_o; e += 1024) XO[(e / pad_o) * xo_pitch + total + e % pad_o] = 0;
}

// The small-batch X pass past kOneMaxElems, in two wide launches over 512-column slabs
// (64 chunks of 8 columns).  M <= 128 rows, so the workgroup of a slab sees every row of its
// columns: which of them are outlier columns is known there exactly, and so are its rows'
// maxima over the other columns.
//   detect_slab (one workgroup of 16 waves per slab, 1 to 8 rows per wave held in
//     registers): the slab's bitmap words and, per row, the slab's largest magnitude
//     pattern over its non-outlier columns (pmax);
//   code_slab (one workgroup per slab and 4 rows, a wave per row): the rows' maxima (max
//     over the slabs' pmax), the slab's outlier ranks (popcounts of the words before it, a
//     scan within it), its part of O, n_O (slab 0), then the codes, X_O and the padding,
//     and (Xqb not NULL, 8 rows or more) the codes again in the product kernel's 1 KB
//     blocks (xqb_offset), zero from K up to the block edge.  When the tiled product kernel
//     follows (up to 112 rows), rows of W_O gather workgroups come first in this launch.
// Both read X (the second time mostly from the cache); together they replace a detection
// launch with too few threads to hide its latency and a one-workgroup-per-row coding.

// A raw buffer resource over [base, base + bytes): loads past the end read 0, so the slab
// kernels issue every load unconditionally and their waits count exactly.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t span_rsrc(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, 0x00020000);
}

template <int DT, int RPW>
__global__ __launch_bounds__(1024) void detect_slab_kernel(const uint16_t* __restrict__ X, int64_t M, int64_t K,
                                                           float tau, uint32_t* __restrict__ bitmap,
                                                           uint32_t* __restrict__ pmax, int64_t nslab) {
    // 16 waves; lane: chunk c of the slab; wave w: rows w, w + 16, ... (RPW of them, M <=
    // 16 RPW).  Rows past M repeat the last row, which changes neither the outlier bits nor
    // a stored maximum.
    __shared__ uint32_t omask[64];
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t c = (int64_t)blockIdx.x * 64 + lane, C = K / 8;
    const bool live = c < C;
    const uint16_t* col = X + (live ? c : C - 1) * 8;
    u32x4 v[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int64_t r = w + 16 * i;
        v[i] = *(const u32x4*)(col + (r < M ? r : M - 1) * K);
    }
    __builtin_amdgcn_sched_barrier(0);  // every load in flight before the first use
    if (threadIdx.x < 64) omask[threadIdx.x] = 0;
    __syncthreads();
    // the chunk's outlier bits: |x| > tau in any row, compared in fp32
    uint32_t mask = 0;
#pragma unroll
    for (int i = 0; i < RPW; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
            mask |= (__builtin_fabsf(to_f32<DT>((uint16_t)(v[i][j >> 1] >> (16 * (j & 1))))) > tau ? 1u : 0u) << j;
    if (mask && live) atomicOr(&omask[lane], mask);
    __syncthreads();
    mask = omask[lane];
    if (w == 0) {
        uint32_t word = mask << (8 * (lane & 3));
        word |= __shfl_xor(word, 1, kWave);
        word |= __shfl_xor(word, 2, kWave);
        // a word's first chunk exists whenever the word does (K % 8 == 0)
        if ((lane & 3) == 0 && live) bitmap[c >> 2] = word;
    }
    // per row, the slab's maximum magnitude pattern over the non-outlier columns
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const u16x2 mb = absmax_bits(u16x2{0, 0}, v[i], mask, true);
        uint32_t m = live ? (mb[0] > mb[1] ? mb[0] : mb[1]) : 0u;
        m = (uint32_t)wave_max((float)m);  // patterns below 2^15 are exact floats
        const int64_t r = w + 16 * i;
        if (lane == 0 && r < M) pmax[r * nslab + blockIdx.x] = m;
    }
}

template <int DT>
__global__ __launch_bounds__(256) void code_slab_kernel(const uint16_t* __restrict__ X, int64_t M, int64_t K,
                                                        const uint32_t* __restrict__ bitmap,
                                                        const uint32_t* __restrict__ pmax, int64_t nslab,
                                                        int32_t* __restrict__ O, int32_t* __restrict__ n_out,
                                                        int8_t* __restrict__ Xq, int64_t xq_pitch,
                                                        int8_t* __restrict__ Xqb, int64_t nsteps,
                                                        float* __restrict__ s_x, uint16_t* __restrict__ XO,
                                                        int64_t xo_pitch, const int8_t* __restrict__ Wq, int64_t N,
                                                        uint16_t* __restrict__ WO, int64_t ny_wo,
                                                        int32_t* __restrict__ zero, int64_t n_zero) {
    __shared__ float inv_s[4];
    __shared__ int32_t wr[16];
    __shared__ uint32_t wb[16];
    __shared__ int32_t tot;
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int64_t sl = blockIdx.x, C = K / 8, Cp = xq_pitch / 8, Kw = ceil_div(K, 32);
    if ((int64_t)blockIdx.y < ny_wo) {
        // the W_O gather (tiled product): 64 rows of Wq per workgroup, O[t] found from the
        // bitmap (the coding workgroups write O meanwhile); workgroup 0 zeroes the counters
        // (a very wide weight: each takes every nb-th group of 64 rows)
        extern __shared__ uint32_t dyn_lds[];
        __shared__ int32_t wsum[4];
        const int64_t b = (int64_t)blockIdx.y * gridDim.x + blockIdx.x, nb = ny_wo * (int64_t)gridDim.x;
        if (b == 0)
            for (int64_t i = tid; i < n_zero; i += 256) zero[i] = 0;
        if (b * 64 >= N) return;
        uint32_t* bits = dyn_lds;
        int32_t* wrank = (int32_t*)(dyn_lds + Kw);
        const int32_t nO = bitmap_ranks(bitmap, Kw, bits, wrank, wsum);
        for (int64_t n0 = b * 64; n0 < N; n0 += nb * 64)
            gather_wo_rows<DT>(n0, K, nO, [&](int32_t t) { return outlier_column(t, Kw, bits, wrank); }, Wq, N, WO,
                               xo_pitch);
        return;
    }
    const int64_t ry = (int64_t)blockIdx.y - ny_wo;  // this workgroup's group of 4 rows
    const int64_t c = sl * 64 + lane, r = ry * 4 + w;  // this thread's chunk and row
    const bool live = c < C, row = r < M;
    // every load first (rows past M, slabs past nslab and chunks past K read 0): the chunk,
    // row r's slab partials (nslab <= 64 kParts), and in wave 0 the bitmap (Kw <= 64 kWords)
    constexpr int kParts = (int)(kSmallK / 512 / 64), kWords = (int)(kSmallK / 32 / 64);
    const __amdgpu_buffer_rsrc_t xr = span_rsrc(X + (row ? r : 0) * K, row ? 2 * K : 0);
    const __amdgpu_buffer_rsrc_t pr = span_rsrc(pmax + (row ? r : 0) * nslab, row ? 4 * nslab : 0);
    const __amdgpu_buffer_rsrc_t br = span_rsrc(bitmap, 4 * Kw);
    const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, (uint32_t)(16 * c), 0, 0));
    uint32_t pm[kParts];
#pragma unroll
    for (int i = 0; i < kParts; ++i) pm[i] = __builtin_amdgcn_raw_buffer_load_b32(pr, (uint32_t)(4 * (lane + 64 * i)), 0, 0);
    uint32_t bw[kWords], wd = 0;
    if (w == 0) {
#pragma unroll
        for (int q = 0; q < kWords; ++q)
            bw[q] = __builtin_amdgcn_raw_buffer_load_b32(br, (uint32_t)(4 * (lane + 64 * q)), 0, 0);
        wd = __builtin_amdgcn_raw_buffer_load_b32(br, (uint32_t)(4 * (16 * sl + lane)), 0, 0);
    }
    // wave w: row r's maximum over the slabs' partials, and its factor
    {
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < kParts; ++i) m = pm[i] > m ? pm[i] : m;
        m = (uint32_t)wave_max((float)m);
        if (lane == 0) {
            const float sv = to_f32<DT>((uint16_t)m);
            inv_s[w] = inv_scale(sv);
            if (row && sl == 0) s_x[r] = sv;
        }
    }
    // wave 0: outlier columns before the slab and in all, the slab's 16 word ranks, its part
    // of O, and n_O
    if (w == 0) {
        int32_t before = 0, all = 0;
#pragma unroll
        for (int q = 0; q < kWords; ++q) {
            const int32_t pc = __popc(bw[q]);
            all += pc;
            before += lane + 64 * q < 16 * sl ? pc : 0;
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            all += __shfl_xor(all, off, kWave);
            before += __shfl_xor(before, off, kWave);
        }
        const int64_t wi = 16 * sl + lane;
        wd = lane < 16 ? wd : 0u;
        const int32_t cnt = __popc(wd);
        int32_t incl = cnt;
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) {
            const int32_t t = __shfl_up(incl, off, kWave);
            if (lane >= off) incl += t;
        }
        if (lane < 16) {
            wr[lane] = before + incl - cnt;
            wb[lane] = wd;
            if (ry == 0) {
                int32_t t = before + incl - cnt;
                for (uint32_t b = wd; b; b &= b - 1) O[t++] = (int32_t)(32 * wi + __ffs(b) - 1);
            }
        }
        if (lane == 0) {
            tot = all;
            if (sl == 0 && ry == 0) *n_out = all;
        }
    }
    __syncthreads();
    const int32_t total = tot, P = (total + 31) & ~31;
    if (row) {
        if (live) {
            wd = wb[(c >> 2) - 16 * sl];
            const uint32_t o = (wd >> (8 * (c & 3))) & 0xffu;
            const u32x2 q = code_chunk<DT>(v, o, inv_s[w], o != 0u);
            *(u32x2*)(Xq + r * xq_pitch + 8 * c) = q;
            if (Xqb) *(u32x2*)(Xqb + xqb_offset(r, 8 * c, nsteps)) = q;
            if (o) {
                int32_t t = wr[(c >> 2) - 16 * sl] + __popc(wd & ((1u << (8 * (c & 3))) - 1u));
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if ((o >> j) & 1u) XO[r * xo_pitch + t++] = (uint16_t)(v[j >> 1] >> (16 * (j & 1)));
            }
        } else if (c < Cp) {
            *(u32x2*)(Xq + r * xq_pitch + 8 * c) = u32x2{0u, 0u};
            if (Xqb && c < 8 * nsteps) *(u32x2*)(Xqb + xqb_offset(r, 8 * c, nsteps)) = u32x2{0u, 0u};
        }
        if (sl == 0)
            for (int32_t t = total + lane; t < P; t += 64) XO[r * xo_pitch + t] = 0;
    }
}

template <int DT, int HOLD>
static hipError_t code_rows_launch1(const XPassArgs& a, const uint32_t* bitmap, int32_t* O, int32_t* n_out,
                                    int64_t n_wo, hipStream_t stream) {
    // persistent row workgroups: as many as fit on the device at once (at most M).  Rows of
    // more than 16384 elements (HOLD 12 or 16) take one workgroup each instead, which measured
    // faster at every batch tried (K = 28672: 246 -> 237 us at M = 8192, 136 -> 132 us at
    // M = 4096), while at K = 12288 the persistent form stays about 1 us ahead.
    const size_t lds = (size_t)ceil_div(a.K, 32) * 8;
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, code_rows_kernel<DT, HOLD>, 256, lds);
    if (e != hipSuccess) return e;
    int64_t groups = HOLD > 8 ? a.M : (int64_t)cus * (per_cu > 0 ? per_cu : 1);
    groups = groups < a.M ? groups : a.M;
    const unsigned grid = (unsigned)(n_wo + groups);
    if (grid == 0) return hipSuccess;
    code_rows_kernel<DT, HOLD><<<grid, 256, lds, stream>>>(
        (const uint16_t*)a.X, a.M, a.K, bitmap, O, n_out, a.Xq, a.xq_pitch, a.s_x, (uint16_t*)a.XO, a.xo_pitch, a.Wq,
        a.N, (uint16_t*)a.WO, n_wo, groups);
    return hipGetLastError();
}

// The register hold is sized to the row (16-byte chunks per thread of 256): fewer
// registers per thread leave room for more workgroups per CU.  Holds of 6 chunks for rows
// of 12288 elements (74 registers, six workgroups per CU, against 84 and five with 8) and
// of 2 for 4096: X pass 62.0 -> 58.9 us on 4096 x 12288, 23.2 -> 22.3 us on 2048 x 4096
// (cold, interleaved on one box, three rounds).
template <int DT>
static hipError_t code_rows_launch(const XPassArgs& a, const uint32_t* bitmap, int32_t* O, int32_t* n_out,
                                   int64_t n_wo, hipStream_t stream) {
    if (a.K <= 2048 * 2) return code_rows_launch1<DT, 2>(a, bitmap, O, n_out, n_wo, stream);
    if (a.K <= 2048 * 4) return code_rows_launch1<DT, 4>(a, bitmap, O, n_out, n_wo, stream);
    if (a.K <= 2048 * 6) return code_rows_launch1<DT, 6>(a, bitmap, O, n_out, n_wo, stream);
    if (a.K <= 2048 * 8) return code_rows_launch1<DT, 8>(a, bitmap, O, n_out, n_wo, stream);
    if (a.K <= 2048 * 12) return code_rows_launch1<DT, 12>(a, bitmap, O, n_out, n_wo, stream);
    if (a.K <= 2048 * 16) return code_rows_launch1<DT, 16>(a, bitmap, O, n_out, n_wo, stream);
    return code_rows_launch1<DT, 0>(a, bitmap, O, n_out, n_wo, stream);
}

// Big path: after detect + compact (which wrote the bitmap, O and n_O).
hipError_t launch_code_rows(const XPassArgs& a, const uint32_t* bitmap, int32_t* O, int32_t* n_out,
                            hipStream_t stream) {
    const int64_t n_wo = a.Wq ? ceil_div(a.N, 64) : 0;
    if (a.M + n_wo == 0) return hipSuccess;
    if (a.dt == F16) return code_rows_launch<F16>(a, bitmap, O, n_out, n_wo, stream);
    return code_rows_launch<BF16>(a, bitmap, O, n_out, n_wo, stream);
}

// Small-batch path (M > 0): one workgroup for at most kOneMaxElems elements, else the
// slab detection and the slab coding.  K = 0 takes the coding launch alone (one slab
// workgroup per 4 rows), which writes s_x = 0 and n_O = 0.
hipError_t launch_xpass_small(const XPassArgs& a, int32_t* O, int32_t* n_out, uint32_t* bitmap, uint32_t* pmax,
                              bool with_wo, int32_t* zero, int64_t n_zero, hipStream_t stream) {
    const uint16_t* x = (const uint16_t*)a.X;
    const int64_t nsteps = ceil_div(a.K, 64);  // blocks per row group of the blocked copy
    if (!with_wo && a.K > 0 && a.M * a.K <= kOneMaxElems) {
        if (a.dt == F16)
            xpass_one_kernel<F16><<<1, 1024, 0, stream>>>(x, (int)a.M, (int)a.K, a.tau, bitmap, O, n_out, a.Xq,
                                                          (int)a.xq_pitch, a.Xqb, (int)nsteps, a.s_x,
                                                          (uint16_t*)a.XO, (int)a.xo_pitch);
        else
            xpass_one_kernel<BF16><<<1, 1024, 0, stream>>>(x, (int)a.M, (int)a.K, a.tau, bitmap, O, n_out, a.Xq,
                                                           (int)a.xq_pitch, a.Xqb, (int)nsteps, a.s_x,
                                                           (uint16_t*)a.XO, (int)a.xo_pitch);
        return hipGetLastError();
    }
    const int64_t nslab = ceil_div(a.K / 8, 64);
    if (nslab > 0) {
        const unsigned g1 = (unsigned)nslab;
        if (a.dt == F16) {
            if (a.M <= 16) detect_slab_kernel<F16, 1><<<g1, 1024, 0, stream>>>(x, a.M, a.K, a.tau, bitmap, pmax, nslab);
            else if (a.M <= 32) detect_slab_kernel<F16, 2><<<g1, 1024, 0, stream>>>(x, a.M, a.K, a.tau, bitmap, pmax, nslab);
            else if (a.M <= 64) detect_slab_kernel<F16, 4><<<g1, 1024, 0, stream>>>(x, a.M, a.K, a.tau, bitmap, pmax, nslab);
            else detect_slab_kernel<F16, 8><<<g1, 1024, 0, stream>>>(x, a.M, a.K, a.tau, bitmap, pmax, nslab);
        } else {
            if (a.M <= 16) detect_slab_kernel<BF16, 1><<<g1, 1024, 0, stream>>>(x, a.M, a.K, a.tau, bitmap, pmax, nslab);
            else if (a.M <= 32) detect_slab_kernel<BF16, 2><<<g1, 1024, 0, stream>>>(x, a.M, a.K, a.tau, bitmap, pmax, nslab);
            else if (a.M <= 64) detect_slab_kernel<BF16, 4><<<g1, 1024, 0, stream>>>(x, a.M, a.K, a.tau, bitmap, pmax, nslab);
            else detect_slab_kernel<BF16, 8><<<g1, 1024, 0, stream>>>(x, a.M, a.K, a.tau, bitmap, pmax, nslab);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    int64_t gx = ceil_div(a.xq_pitch / 8, 64);
    gx = gx > 0 ? gx : 1;
    // with_wo: rows of gather workgroups first (one per 64 weight rows, at most kMaxGatherRows
    // rows of them: the grid's y extent is limited), then the coding
    constexpr int64_t kMaxGatherRows = 4096;
    int64_t ny_wo = with_wo ? ceil_div(ceil_div(a.N, 64), gx) : 0;
    ny_wo = ny_wo < kMaxGatherRows ? ny_wo : kMaxGatherRows;
    const size_t lds = with_wo ? (size_t)ceil_div(a.K, 32) * 8 : 0;
    const dim3 g2((unsigned)gx, (unsigned)(ny_wo + ceil_div(a.M, 4)));
    if (a.dt == F16)
        code_slab_kernel<F16><<<g2, 256, lds, stream>>>(x, a.M, a.K, bitmap, pmax, nslab, O, n_out, a.Xq, a.xq_pitch,
                                                        a.Xqb, nsteps, a.s_x, (uint16_t*)a.XO, a.xo_pitch, a.Wq, a.N,
                                                        (uint16_t*)a.WO, ny_wo, zero, n_zero);
    else
        code_slab_kernel<BF16><<<g2, 256, lds, stream>>>(x, a.M, a.K, bitmap, pmax, nslab, O, n_out, a.Xq, a.xq_pitch,
                                                         a.Xqb, nsteps, a.s_x, (uint16_t*)a.XO, a.xo_pitch, a.Wq, a.N,
                                                         (uint16_t*)a.WO, ny_wo, zero, n_zero);
    return hipGetLastError();
}

}  // namespace llmint8
