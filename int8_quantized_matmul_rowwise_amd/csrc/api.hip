// C-ABI entry points of llmint8 (declared and documented in include/llmint8.h).
// Validation happens before anything is enqueued; HIP failures map to LLMINT8_EHIP.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "../../include/llmint8.h"
#include "common.hpp"
#include "launch.hpp"

#define LLMINT8_API extern "C" __attribute__((visibility("default")))

using namespace llmint8;

namespace {

constexpr int64_t kMaxK = 133143;  // 127 * 127 * K < 2^31
constexpr int64_t kMaxDim = 0x7fffffff;
constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

// Shape rules shared by every call (see the header).
int check_shape(int64_t M, int64_t K, int64_t N, int dtype) {
    if (dtype != LLMINT8_F16 && dtype != LLMINT8_BF16) return LLMINT8_EINVAL;
    if (M < 0 || K < 0 || N < 0 || M > kMaxDim || N > kMaxDim) return LLMINT8_EINVAL;
    if (K % 16 != 0 || N % 8 != 0) return LLMINT8_EINVAL;
    if (K > kMaxK) return LLMINT8_ERANGE;
    if (ceil_div(M, 256) * ceil_div(N, 256) > kMaxDim) return LLMINT8_ERANGE;
    return LLMINT8_OK;
}

int check_threshold(float t) { return (isnan(t) || t < 0.0f) ? LLMINT8_EINVAL : LLMINT8_OK; }

struct Layout {
    size_t xq, xq_pitch, s_x, n_outliers, outliers, xo, xo_pitch, wo, bitmap, partial, pmax, xqb, sk_cnt, sk_part,
        total;
    bool sk;  // the tiled product kernel runs stream-K for these sizes
};

Layout make_layout(int64_t M, int64_t K, int64_t N) {
    Layout L;
    const size_t m = (size_t)M, k = (size_t)K, n = (size_t)N;
    L.xq_pitch = (size_t)round_up(K, 256);
    L.xo_pitch = (size_t)round_up(K, 32);
    const size_t kw = (size_t)ceil_div(K, 32);
    size_t off = 0;
    L.xq = off;
    off = align_up(off + m * L.xq_pitch);
    L.s_x = off;
    off = align_up(off + 4 * m);
    L.n_outliers = off;
    off = align_up(off + 4);
    L.outliers = off;
    off = align_up(off + 4 * k);
    L.xo = off;
    off = align_up(off + 2 * m * L.xo_pitch);
    // W_O: the tiled path's gathered Wq[:,O]; the small-batch kernel gathers it itself
    L.wo = off;
    off = align_up(off + (small_batch(M, K, N) ? 0 : 2 * n * L.xo_pitch));
    L.bitmap = off;
    off = align_up(off + 4 * kw);
    L.partial = off;
    off = align_up(off + 4 * kw * (size_t)detect_row_blocks(M));
    L.pmax = off;  // the slab X pass: per row and 512-column slab, the slab's row maximum
    off = align_up(off + (small_batch(M, K, N) || slab_xpass(M, K) ? 4 * m * (size_t)ceil_div(K, 512) : 0));
    L.xqb = off;  // small batches of 8 rows or more: Xq again, in the product kernel's 1 KB blocks
    const bool blocked = small_batch(M, K, N) && small_blocked_codes(M);
    off = align_up(off + (blocked ? (size_t)round_up(M, 16) * (size_t)ceil_div(K, 64) * 64 : 0));
    // stream-K (tiled path, few tiles): a counter per tile, two partial tiles per workgroup
    L.sk = stream_k_shape(M, K, N);
    L.sk_cnt = off;
    off = align_up(off + (L.sk ? 4 * (size_t)gemm_tiles(M, N) : 0));
    L.sk_part = off;
    off = align_up(off + (L.sk ? 2 * (size_t)stream_k_grid(M, K, N) * (size_t)kStreamKSlotBytes : 0));
    L.total = off;
    return L;
}

// ---- failure injection and logging (host layer only; both read the environment per call)
//   LLMINT8_FAULT=<stage>  dry run: nothing is enqueued; every stage the call reaches before
//                          the named one counts as done, the named one as failed, so the
//                          error path (LLMINT8_EHIP, nothing reported as done) runs on a
//                          machine without a GPU.  A call whose path does not contain the
//                          stage returns LLMINT8_OK having enqueued nothing.
//   LLMINT8_LOG=1          each call's sizes, dtype, threshold and path, and each stage, on
//                          stderr.
const char* fault_stage() {
    const char* f = getenv("LLMINT8_FAULT");
    return f && *f ? f : nullptr;
}

bool log_on() {
    const char* l = getenv("LLMINT8_LOG");
    return l && *l && strcmp(l, "0") != 0;
}

const char* dtype_name(int dt) { return dt == LLMINT8_F16 ? "fp16" : "bf16"; }

// tau: NaN where the call takes no threshold
void log_call(const char* fn, int64_t M, int64_t K, int64_t N, int dt, float tau, const char* path) {
    if (!log_on()) return;
    char t[32] = "";
    if (!isnan(tau)) snprintf(t, sizeof t, " threshold=%g", (double)tau);
    fprintf(stderr, "[llmint8] %s M=%lld K=%lld N=%lld dtype=%s%s path=%s%s\n", fn, (long long)M, (long long)K,
            (long long)N, dtype_name(dt), t, path, fault_stage() ? " (dry run)" : "");
}

// Run one stage of a call: `launch` enqueues it and returns its HIP status.
template <class Launch>
hipError_t stage(const char* name, Launch&& launch) {
    const char* f = fault_stage();
    const bool fail = f && strcmp(f, name) == 0;
    if (log_on()) fprintf(stderr, "[llmint8]   stage %s%s\n", name, fail ? ": injected failure" : (f ? ": skipped" : ""));
    if (f) return fail ? hipErrorLaunchFailure : hipSuccess;
    return launch();
}

int hip_status(hipError_t e) {
    if (e == hipSuccess) return LLMINT8_OK;
    if (!fault_stage()) (void)hipGetLastError();  // consume the sticky error (an injected one has none)
    return LLMINT8_EHIP;
}

// Enqueue the X pass into the workspace: on the small-batch path its own launches; on the
// tiled path detect, compact and the row coding (+ the W_O gather).
int run_xpass(const void* X, int64_t M, int64_t K, int dtype, float tau, const int8_t* Wq, int64_t N,
              int8_t* ws, const Layout& L, hipStream_t st) {
    uint32_t* partial = (uint32_t*)(ws + L.partial);
    uint32_t* bitmap = (uint32_t*)(ws + L.bitmap);
    int32_t* O = (int32_t*)(ws + L.outliers);
    int32_t* nO = (int32_t*)(ws + L.n_outliers);
    XPassArgs a{};
    a.dt = dtype;
    a.X = X;
    a.tau = tau;
    a.M = M;
    a.K = K;
    a.N = N;
    a.Xq = ws + L.xq;
    a.xq_pitch = (int64_t)L.xq_pitch;
    a.s_x = (float*)(ws + L.s_x);
    a.XO = ws + L.xo;
    a.xo_pitch = (int64_t)L.xo_pitch;
    if (small_batch(M, K, N)) {
        a.Xqb = small_blocked_codes(M) ? ws + L.xqb : nullptr;
        return hip_status(stage("xpass_small", [&] {
            return launch_xpass_small(a, O, nO, bitmap, (uint32_t*)(ws + L.pmax), false, nullptr, 0, st);
        }));
    }
    a.Xqb = nullptr;
    int32_t* sk_cnt = L.sk ? (int32_t*)(ws + L.sk_cnt) : nullptr;  // zeroed for the product kernel
    const int64_t n_tiles = gemm_tiles(M, N);
    if (slab_xpass(M, K)) {
        a.Wq = Wq;
        a.WO = ws + L.wo;
        return hip_status(stage("xpass_small", [&] {
            return launch_xpass_small(a, O, nO, bitmap, (uint32_t*)(ws + L.pmax), Wq != nullptr, sk_cnt,
                                      sk_cnt ? n_tiles : 0, st);
        }));
    }
    hipError_t e = stage("detect", [&] { return launch_detect(dtype, X, M, K, tau, partial, st); });
    if (e == hipSuccess)
        e = stage("compact", [&] { return launch_compact(M, K, partial, bitmap, O, nO, st, sk_cnt, n_tiles); });
    if (e == hipSuccess) {
        a.M = M;
        a.K = K;
        a.N = N;
        a.bitmap = bitmap;
        a.O = O;
        a.n_out = nO;
        a.Xq = ws + L.xq;
        a.xq_pitch = (int64_t)L.xq_pitch;
        a.s_x = (float*)(ws + L.s_x);
        a.XO = ws + L.xo;
        a.xo_pitch = (int64_t)L.xo_pitch;
        a.Wq = Wq;
        a.WO = ws + L.wo;
        e = stage("code_rows", [&] { return launch_code_rows(a, bitmap, O, nO, st); });
    }
    return hip_status(e);
}

// Each stage validates its arguments and, when `enqueue` is set and they are valid,
// enqueues its kernels.
int prepare_common(const void* X, int64_t M, int64_t K, int dtype, const int8_t* Wq, int64_t N, float threshold,
                   void* workspace, size_t workspace_bytes, void* stream, bool enqueue) {
    int rc = check_shape(M, K, N, dtype);
    if (rc) return rc;
    if ((rc = check_threshold(threshold))) return rc;
    if (M > 0 && K > 0 && (!X || !aligned(X, 16))) return LLMINT8_EINVAL;
    if (M > 0 && N > 0 && K > 0 && (!Wq || !aligned(Wq, 16))) return LLMINT8_EINVAL;
    const Layout L = make_layout(M, K, N);
    if (M > 0 && (!workspace || !aligned(workspace, 16) || workspace_bytes < L.total)) return LLMINT8_EWORKSPACE;
    if (overlap(workspace, L.total, X, (size_t)M * (size_t)K * 2) ||
        overlap(workspace, L.total, Wq, (size_t)N * (size_t)K))
        return LLMINT8_EINVAL;
    if (M == 0 || !enqueue) return LLMINT8_OK;
    log_call("x pass", M, K, N, dtype, threshold, small_batch(M, K, N) ? "small_batch" : "tiled");
    return run_xpass(X, M, K, dtype, threshold, N > 0 ? Wq : nullptr, N, (int8_t*)workspace, L,
                     (hipStream_t)stream);
}

// Products + epilogue (Y != NULL) or the accumulator dump (C, F) from a prepared workspace.
int products_common(int64_t M, int64_t K, int dtype, const int8_t* Wq, const float* w_scale, int64_t N, void* Y,
                    int32_t* C, float* F, void* workspace, size_t workspace_bytes, void* stream,
                    bool enqueue, const void* WO_fixed = nullptr, int64_t wo_pitch_fixed = 0) {
    int rc = check_shape(M, K, N, dtype);
    if (rc) return rc;
    const bool acc = Y == nullptr;
    if (M > 0 && N > 0) {
        if (K > 0 && (!Wq || !aligned(Wq, 16))) return LLMINT8_EINVAL;
        if (acc) {
            if (!C || !F || !aligned(C, 16) || !aligned(F, 16)) return LLMINT8_EINVAL;
        } else if (!Y || !aligned(Y, 16) || !w_scale || !aligned(w_scale, 4)) {
            return LLMINT8_EINVAL;
        }
    }
    const Layout L = make_layout(M, K, N);
    if (M > 0 && (!workspace || !aligned(workspace, 16) || workspace_bytes < L.total)) return LLMINT8_EWORKSPACE;
    if (!acc) {
        const size_t yb = (size_t)M * (size_t)N * 2;
        if (overlap(Y, yb, Wq, (size_t)N * (size_t)K) || overlap(Y, yb, w_scale, (size_t)N * 4) ||
            overlap(Y, yb, workspace, L.total))
            return LLMINT8_EINVAL;
    }
    if (M == 0 || N == 0 || !enqueue) return LLMINT8_OK;
    log_call(acc ? "products (accumulator dump)" : (WO_fixed ? "products (fixed outlier set)" : "products"), M, K, N,
             dtype, NAN, small_batch(M, K, N) ? "small_batch" : (L.sk ? "tiled_stream_k" : "tiled"));
    int8_t* ws = (int8_t*)workspace;
    GemmArgs g;
    g.dt = dtype;
    g.Xq = ws + L.xq;
    g.xq_pitch = (int64_t)L.xq_pitch;
    g.Wq = Wq;
    g.M = M;
    g.N = N;
    g.K = K;
    g.s_x = (const float*)(ws + L.s_x);
    g.s_w = w_scale;
    g.XO = ws + L.xo;
    g.xo_pitch = (int64_t)L.xo_pitch;
    g.f_scaled = WO_fixed == nullptr;
    g.WO = g.f_scaled ? (const void*)(ws + L.wo) : WO_fixed;
    g.wo_pitch = g.f_scaled ? (int64_t)L.xo_pitch : wo_pitch_fixed;
    g.n_out = (const int32_t*)(ws + L.n_outliers);
    g.O = (const int32_t*)(ws + L.outliers);
    g.Y = Y;
    g.C_acc = C;
    g.F_acc = F;
    g.sk_cnt = L.sk ? (int32_t*)(ws + L.sk_cnt) : nullptr;
    g.sk_part = L.sk ? (int32_t*)(ws + L.sk_part) : nullptr;
    // the small-batch X pass writes the blocked copy; the fixed-set X pass (row coding) does not
    g.Xqb = !WO_fixed && small_blocked_codes(M) ? ws + L.xqb : nullptr;
    if (small_batch(M, K, N)) return hip_status(stage("gemm_small", [&] { return launch_gemm_small(g, (hipStream_t)stream); }));
    return hip_status(stage("gemm", [&] { return launch_gemm(g, (hipStream_t)stream); }));
}

// X pass against a caller's fixed outlier set: its bitmap (as one partial), the
// compaction (O, n_O in the workspace), then the row coding; no W_O gather.
int run_xpass_fixed(const void* X, int64_t M, int64_t K, int64_t N, int dtype, const int32_t* Ofix, int64_t nO,
                    int8_t* ws, const Layout& L, hipStream_t st) {
    uint32_t* partial = (uint32_t*)(ws + L.partial);
    uint32_t* bitmap = (uint32_t*)(ws + L.bitmap);
    int32_t* O = (int32_t*)(ws + L.outliers);
    int32_t* n_out = (int32_t*)(ws + L.n_outliers);
    int32_t* sk_cnt = L.sk ? (int32_t*)(ws + L.sk_cnt) : nullptr;  // zeroed for the product kernel
    const int64_t n_tiles = gemm_tiles(M, N);
    hipError_t e = stage("list_bitmap", [&] { return launch_list_bitmap(K, Ofix, nO, partial, st); });
    if (e == hipSuccess)
        e = stage("compact", [&] { return launch_compact(1, K, partial, bitmap, O, n_out, st, sk_cnt, n_tiles); });
    if (e == hipSuccess) {
        XPassArgs a{};
        a.dt = dtype;
        a.X = X;
        a.tau = 0.0f;
        a.M = M;
        a.K = K;
        a.N = 0;
        a.bitmap = bitmap;
        a.O = O;
        a.n_out = n_out;
        a.Xq = ws + L.xq;
        a.xq_pitch = (int64_t)L.xq_pitch;
        a.Xqb = nullptr;
        a.s_x = (float*)(ws + L.s_x);
        a.XO = ws + L.xo;
        a.xo_pitch = (int64_t)L.xo_pitch;
        a.Wq = nullptr;
        a.WO = nullptr;
        e = stage("code_rows", [&] { return launch_code_rows(a, bitmap, O, n_out, st); });
    }
    return hip_status(e);
}

int64_t fixed_pitch(int64_t nO) { return (nO + 31) / 32 * 32; }

int matmul_common(const void* X, int64_t M, int64_t K, int dtype, const int8_t* Wq, const float* w_scale,
                  int64_t N, float threshold, void* Y, int32_t* C, float* F, void* workspace,
                  size_t workspace_bytes, void* stream, bool enqueue = true) {
    // validate both stages before enqueueing either
    int rc = prepare_common(X, M, K, dtype, Wq, N, threshold, workspace, workspace_bytes, stream, false);
    if (rc) return rc;
    rc = products_common(M, K, dtype, Wq, w_scale, N, Y, C, F, workspace, workspace_bytes, stream, false);
    if (rc) return rc;
    if (Y && overlap(Y, (size_t)M * (size_t)N * 2, X, (size_t)M * (size_t)K * 2)) return LLMINT8_EINVAL;
    if (!enqueue) return LLMINT8_OK;
    rc = prepare_common(X, M, K, dtype, Wq, N, threshold, workspace, workspace_bytes, stream, true);
    if (rc) return rc;
    return products_common(M, K, dtype, Wq, w_scale, N, Y, C, F, workspace, workspace_bytes, stream, true);
}

}  // namespace

LLMINT8_API const char* llmint8_status_string(int status) {
    switch (status) {
        case LLMINT8_OK: return "LLMINT8_OK";
        case LLMINT8_EINVAL: return "LLMINT8_EINVAL: invalid argument";
        case LLMINT8_EWORKSPACE: return "LLMINT8_EWORKSPACE: workspace missing, misaligned or too small";
        case LLMINT8_EHIP: return "LLMINT8_EHIP: HIP runtime or launch failure";
        case LLMINT8_ERANGE: return "LLMINT8_ERANGE: size outside the exact-int32 range";
        default: return "LLMINT8: unknown status";
    }
}

LLMINT8_API int int8_quantize_weight(const void* W, int64_t K, int64_t N, int dtype, int8_t* Wq, float* w_scale,
                                     void* stream) {
    int rc = check_shape(0, K, N, dtype);
    if (rc) return rc;
    if (N == 0) return LLMINT8_OK;
    if (!w_scale || !aligned(w_scale, 4)) return LLMINT8_EINVAL;
    if (K > 0 && (!W || !Wq || !aligned(W, 16) || !aligned(Wq, 16))) return LLMINT8_EINVAL;
    if (overlap(W, (size_t)K * N * 2, Wq, (size_t)K * N) || overlap(W, (size_t)K * N * 2, w_scale, (size_t)N * 4) ||
        overlap(Wq, (size_t)K * N, w_scale, (size_t)N * 4))
        return LLMINT8_EINVAL;
    log_call("int8_quantize_weight", 0, K, N, dtype, NAN, "weight");
    return hip_status(stage("weight", [&] { return launch_weight(dtype, W, K, N, Wq, w_scale, nullptr, (hipStream_t)stream); }));
}

LLMINT8_API size_t int8_matmul_workspace_bytes(int64_t M, int64_t K, int64_t N) {
    if (M < 0 || K < 0 || N < 0) return 0;
    return make_layout(M, K, N).total;
}

LLMINT8_API int int8_matmul_workspace_layout(int64_t M, int64_t K, int64_t N, llmint8_workspace_layout* out) {
    if (!out || M < 0 || K < 0 || N < 0) return LLMINT8_EINVAL;
    const Layout L = make_layout(M, K, N);
    out->xq = L.xq;
    out->xq_pitch = L.xq_pitch;
    out->s_x = L.s_x;
    out->n_outliers = L.n_outliers;
    out->outliers = L.outliers;
    out->xo = L.xo;
    out->xo_pitch = L.xo_pitch;
    out->wo = L.wo;
    out->scratch = L.bitmap;
    out->total = L.total;
    out->small_batch = small_batch(M, K, N) ? 1 : 0;
    return LLMINT8_OK;
}

LLMINT8_API int int8_matmul(const void* X, int64_t M, int64_t K, int dtype, const int8_t* Wq,
                            const float* w_scale, int64_t N, float threshold, void* Y, void* workspace,
                            size_t workspace_bytes, void* stream) {
    if (!Y && M > 0 && N > 0) return LLMINT8_EINVAL;
    return matmul_common(X, M, K, dtype, Wq, w_scale, N, threshold, Y, nullptr, nullptr, workspace,
                         workspace_bytes, stream);
}

LLMINT8_API int int8_matmul_accumulators(const void* X, int64_t M, int64_t K, int dtype, const int8_t* Wq,
                                         int64_t N, float threshold, int32_t* C, float* F, void* workspace,
                                         size_t workspace_bytes, void* stream) {
    if ((!C || !F) && M > 0 && N > 0) return LLMINT8_EINVAL;
    return matmul_common(X, M, K, dtype, Wq, nullptr, N, threshold, nullptr, C, F, workspace, workspace_bytes,
                         stream);
}

LLMINT8_API int int8_matmul_stats(const void* X, int64_t M, int64_t K, int dtype, float threshold,
                                  int32_t* n_outlier_cols, int32_t* outlier_cols, void* workspace,
                                  size_t workspace_bytes, void* stream) {
    int rc = check_shape(M, K, 0, dtype);
    if (rc) return rc;
    if ((rc = check_threshold(threshold))) return rc;
    if (!n_outlier_cols) return LLMINT8_EINVAL;
    if (M > 0 && K > 0 && (!X || !aligned(X, 16))) return LLMINT8_EINVAL;
    if (outlier_cols && !aligned(outlier_cols, 4)) return LLMINT8_EINVAL;
    const Layout L = make_layout(M, K, 0);
    if (M > 0 && (!workspace || !aligned(workspace, 16) || workspace_bytes < L.total)) return LLMINT8_EWORKSPACE;
    if (M == 0 || K == 0) {
        *n_outlier_cols = 0;
        return LLMINT8_OK;
    }
    hipStream_t st = (hipStream_t)stream;
    int8_t* ws = (int8_t*)workspace;
    log_call("int8_matmul_stats", M, K, 0, dtype, threshold, "detect");
    hipError_t e = stage("detect", [&] { return launch_detect(dtype, X, M, K, threshold, (uint32_t*)(ws + L.partial), st); });
    if (e == hipSuccess)
        e = stage("compact", [&] {
            return launch_compact(M, K, (const uint32_t*)(ws + L.partial), (uint32_t*)(ws + L.bitmap),
                                  (int32_t*)(ws + L.outliers), (int32_t*)(ws + L.n_outliers), st);
        });
    int32_t n = 0;
    if (e == hipSuccess)
        e = stage("stats_copy", [&] { return hipMemcpyAsync(&n, ws + L.n_outliers, 4, hipMemcpyDeviceToHost, st); });
    if (e == hipSuccess) e = stage("stats_sync", [&] { return hipStreamSynchronize(st); });
    if (e == hipSuccess && outlier_cols && (n > 0 || fault_stage())) {
        e = stage("stats_copy_cols", [&] {
            hipError_t c = hipMemcpyAsync(outlier_cols, ws + L.outliers, (size_t)n * 4, hipMemcpyDeviceToDevice, st);
            return c == hipSuccess ? hipStreamSynchronize(st) : c;
        });
    }
    if (e != hipSuccess) return hip_status(e);  // *n_outlier_cols is left as it was
    *n_outlier_cols = n;
    return LLMINT8_OK;
}

LLMINT8_API int int8_matmul_prepare(const void* X, int64_t M, int64_t K, int dtype, const int8_t* Wq, int64_t N,
                                    float threshold, void* workspace, size_t workspace_bytes, void* stream) {
    return prepare_common(X, M, K, dtype, Wq, N, threshold, workspace, workspace_bytes, stream, true);
}

LLMINT8_API int int8_matmul_products(int64_t M, int64_t K, int dtype, const int8_t* Wq, const float* w_scale,
                                     int64_t N, void* Y, void* workspace, size_t workspace_bytes,
                                     void* stream) {
    if (!Y && M > 0 && N > 0) return LLMINT8_EINVAL;
    return products_common(M, K, dtype, Wq, w_scale, N, Y, nullptr, nullptr, workspace, workspace_bytes, stream,
                           true);
}

// ---- block-wise absmax int8 codec

LLMINT8_API int int8_blockwise_quantize(const float* x, int64_t n, int64_t block, int8_t* q, float* absmax,
                                        void* stream) {
    if (n < 0 || !codec_block_ok(block)) return LLMINT8_EINVAL;
    if (n == 0) return LLMINT8_OK;
    const int64_t nb = ceil_div(n, block);
    if (!x || !q || !absmax || !aligned(x, 16) || !aligned(q, 4) || !aligned(absmax, 4)) return LLMINT8_EINVAL;
    if (overlap(x, (size_t)n * 4, q, (size_t)n) || overlap(x, (size_t)n * 4, absmax, (size_t)nb * 4) ||
        overlap(q, (size_t)n, absmax, (size_t)nb * 4))
        return LLMINT8_EINVAL;
    log_call("int8_blockwise_quantize", 0, block, n, LLMINT8_F16, NAN, "codec");
    return hip_status(stage("block_quantize", [&] { return launch_block_quantize(x, n, block, q, absmax, (hipStream_t)stream); }));
}

LLMINT8_API int int8_blockwise_dequantize(const int8_t* q, const float* absmax, int64_t n, int64_t block, float* x,
                                          void* stream) {
    if (n < 0 || !codec_block_ok(block)) return LLMINT8_EINVAL;
    if (n == 0) return LLMINT8_OK;
    const int64_t nb = ceil_div(n, block);
    if (!x || !q || !absmax || !aligned(x, 16) || !aligned(q, 4) || !aligned(absmax, 4)) return LLMINT8_EINVAL;
    if (overlap(x, (size_t)n * 4, q, (size_t)n) || overlap(x, (size_t)n * 4, absmax, (size_t)nb * 4))
        return LLMINT8_EINVAL;
    log_call("int8_blockwise_dequantize", 0, block, n, LLMINT8_F16, NAN, "codec");
    return hip_status(stage("block_dequantize", [&] { return launch_block_dequantize(q, absmax, n, block, x, (hipStream_t)stream); }));
}

// ---- fixed (caller-supplied) outlier dimensions

LLMINT8_API size_t int8_quantize_weight_fixed_workspace_bytes(int64_t K) {
    if (K < 0) return 0;
    return align_up((size_t)ceil_div(K, 32) * 4 + 1);
}

LLMINT8_API int int8_quantize_weight_fixed(const void* W, int64_t K, int64_t N, int dtype, const int32_t* outlier_cols,
                                           int64_t n_outlier_cols, int8_t* Wq, float* w_scale, void* W_O,
                                           void* workspace, size_t workspace_bytes, void* stream) {
    int rc = check_shape(0, K, N, dtype);
    if (rc) return rc;
    const int64_t nO = n_outlier_cols, P = fixed_pitch(nO);
    if (nO < 0 || nO > K) return LLMINT8_EINVAL;
    if (N == 0) return LLMINT8_OK;
    if (!w_scale || !aligned(w_scale, 4)) return LLMINT8_EINVAL;
    if (K > 0 && (!W || !Wq || !aligned(W, 16) || !aligned(Wq, 16))) return LLMINT8_EINVAL;
    if (nO > 0 && (!outlier_cols || !aligned(outlier_cols, 4) || !W_O || !aligned(W_O, 16))) return LLMINT8_EINVAL;
    if (K > 0 && (!workspace || !aligned(workspace, 16) ||
                  workspace_bytes < int8_quantize_weight_fixed_workspace_bytes(K)))
        return LLMINT8_EWORKSPACE;
    const size_t wb = (size_t)K * N * 2, qb = (size_t)K * N, sb = (size_t)N * 4, ob = (size_t)N * P * 2;
    const size_t kb = int8_quantize_weight_fixed_workspace_bytes(K);
    if (overlap(W, wb, Wq, qb) || overlap(W, wb, w_scale, sb) || overlap(Wq, qb, w_scale, sb) ||
        overlap(W_O, ob, W, wb) || overlap(W_O, ob, Wq, qb) || overlap(W_O, ob, w_scale, sb) ||
        overlap(workspace, kb, W, wb) || overlap(workspace, kb, Wq, qb) || overlap(workspace, kb, w_scale, sb) ||
        overlap(workspace, kb, W_O, ob) || overlap(outlier_cols, (size_t)nO * 4, W_O, ob) ||
        overlap(outlier_cols, (size_t)nO * 4, Wq, qb) || overlap(outlier_cols, (size_t)nO * 4, w_scale, sb))
        return LLMINT8_EINVAL;
    hipStream_t st = (hipStream_t)stream;
    uint32_t* skip = (uint32_t*)workspace;
    log_call("int8_quantize_weight_fixed", 0, K, N, dtype, NAN, "weight");
    hipError_t e = stage("list_bitmap", [&] { return launch_list_bitmap(K, outlier_cols, nO, skip, st); });
    if (e == hipSuccess) e = stage("weight", [&] { return launch_weight(dtype, W, K, N, Wq, w_scale, K > 0 ? skip : nullptr, st); });
    if (e == hipSuccess) e = stage("gather_wo", [&] { return launch_gather_wo(W, K, N, outlier_cols, nO, P, W_O, st); });
    return hip_status(e);
}

LLMINT8_API int int8_matmul_fixed(const void* X, int64_t M, int64_t K, int dtype, const int32_t* outlier_cols,
                                  int64_t n_outlier_cols, const int8_t* Wq, const float* w_scale, const void* W_O,
                                  int64_t N, void* Y, void* workspace, size_t workspace_bytes, void* stream) {
    int rc = check_shape(M, K, N, dtype);
    if (rc) return rc;
    const int64_t nO = n_outlier_cols, P = fixed_pitch(nO);
    if (nO < 0 || nO > K) return LLMINT8_EINVAL;
    if (M > 0 && K > 0 && (!X || !aligned(X, 16))) return LLMINT8_EINVAL;
    if (M > 0 && nO > 0 && (!outlier_cols || !aligned(outlier_cols, 4))) return LLMINT8_EINVAL;
    if (M > 0 && N > 0 && nO > 0 && (!W_O || !aligned(W_O, 16))) return LLMINT8_EINVAL;
    const Layout L = make_layout(M, K, N);
    if (M > 0 && (!workspace || !aligned(workspace, 16) || workspace_bytes < L.total)) return LLMINT8_EWORKSPACE;
    if (overlap(workspace, L.total, X, (size_t)M * (size_t)K * 2) ||
        overlap(workspace, L.total, Wq, (size_t)N * (size_t)K) ||
        overlap(workspace, L.total, outlier_cols, (size_t)nO * 4) ||
        overlap(workspace, L.total, W_O, (size_t)N * P * 2))
        return LLMINT8_EINVAL;
    rc = products_common(M, K, dtype, Wq, w_scale, N, Y, nullptr, nullptr, workspace, workspace_bytes, stream, false,
                         W_O, P);
    if (rc) return rc;
    if (Y && (overlap(Y, (size_t)M * (size_t)N * 2, X, (size_t)M * (size_t)K * 2) ||
              overlap(Y, (size_t)M * (size_t)N * 2, W_O, (size_t)N * P * 2) ||
              overlap(Y, (size_t)M * (size_t)N * 2, outlier_cols, (size_t)nO * 4)))
        return LLMINT8_EINVAL;
    if (M == 0) return LLMINT8_OK;
    log_call("fixed x pass", M, K, N, dtype, NAN, "fixed");
    rc = run_xpass_fixed(X, M, K, N, dtype, outlier_cols, nO, (int8_t*)workspace, L, (hipStream_t)stream);
    if (rc) return rc;
    return products_common(M, K, dtype, Wq, w_scale, N, Y, nullptr, nullptr, workspace, workspace_bytes, stream, true,
                           W_O, P);
}

// ---- group-wise scales along K

namespace {

struct GroupLayout {
    size_t xq, s_x, rg, xqb, total;
    bool blocked;  // the X pass also writes the blocked copy (xqb) for the small-batch kernel
};

GroupLayout group_layout(int64_t M, int64_t K, int64_t G) {
    GroupLayout L;
    const size_t m = (size_t)M, ng = (size_t)(K / G);
    L.blocked = group_blocked_codes(M, K, G);
    L.xq = 0;
    L.s_x = align_up(m * (size_t)K);
    L.rg = align_up(L.s_x + 4 * m * ng);
    L.xqb = align_up(L.rg + 4 * m * ng);
    L.total = align_up(L.xqb + (L.blocked ? (size_t)round_up(M, 16) * (size_t)K : 0));
    return L;
}

int check_group(int64_t M, int64_t K, int64_t N, int dtype, int64_t G) {
    int rc = check_shape(M, K, N, dtype);
    if (rc) return rc;
    if (K > 0 && !group_size_ok(G, K)) return LLMINT8_EINVAL;
    if (ceil_div(M, 256) * ceil_div(N, 128) > kMaxDim) return LLMINT8_ERANGE;
    return LLMINT8_OK;
}

}  // namespace

LLMINT8_API int int8_quantize_weight_group(const void* W, int64_t K, int64_t N, int dtype, int64_t group, int8_t* Wq,
                                           float* w_scale, void* stream) {
    int rc = check_group(0, K, N, dtype, group);
    if (rc) return rc;
    if (N == 0 || K == 0) return LLMINT8_OK;
    const size_t wb = (size_t)K * N * 2, qb = (size_t)K * N, sb = (size_t)N * (size_t)(K / group) * 4;
    if (!W || !Wq || !w_scale || !aligned(W, 16) || !aligned(Wq, 16) || !aligned(w_scale, 4)) return LLMINT8_EINVAL;
    if (overlap(W, wb, Wq, qb) || overlap(W, wb, w_scale, sb) || overlap(Wq, qb, w_scale, sb)) return LLMINT8_EINVAL;
    hipStream_t st = (hipStream_t)stream;
    log_call("int8_quantize_weight_group", 0, K, N, dtype, NAN, "weight");
    hipError_t e = stage("group_colmax", [&] { return launch_group_colmax(dtype, W, K, N, group, w_scale, st); });
    if (e == hipSuccess)
        e = stage("quantize_weight_groups", [&] { return launch_quantize_weight_groups(dtype, W, K, N, w_scale, group, Wq, st); });
    return hip_status(e);
}

LLMINT8_API size_t int8_matmul_group_workspace_bytes(int64_t M, int64_t K, int64_t group) {
    if (M < 0 || K < 0 || (K > 0 && !group_size_ok(group, K))) return 0;
    if (K == 0) return align_up(0);
    return group_layout(M, K, group).total;
}

namespace {

// int8_matmul_group and its two halves: the X pass (xpass) into the workspace and the
// products (products) from it.
int group_common(const void* X, int64_t M, int64_t K, int dtype, int64_t group, const int8_t* Wq,
                 const float* w_scale, int64_t N, void* Y, void* workspace, size_t workspace_bytes, void* stream,
                 bool xpass, bool products) {
    int rc = check_group(M, K, N, dtype, group);
    if (rc) return rc;
    if (M == 0 || (products && N == 0 && !xpass)) return LLMINT8_OK;
    hipStream_t st = (hipStream_t)stream;
    if (products && N > 0) {
        if (!Y || !aligned(Y, 16)) return LLMINT8_EINVAL;
        if (K == 0) log_call("int8_matmul_group", M, K, N, dtype, NAN, "empty sum");
        if (K == 0)  // the empty sum; N is even
            return hip_status(stage("fill_zero", [&] { return launch_fill_zero((float*)Y, M * N / 2, st); }));
        if (!Wq || !w_scale || !aligned(Wq, 16) || !aligned(w_scale, 4)) return LLMINT8_EINVAL;
    }
    if (K == 0) return LLMINT8_OK;
    if (xpass && (!X || !aligned(X, 16))) return LLMINT8_EINVAL;
    const GroupLayout L = group_layout(M, K, group);
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < L.total) return LLMINT8_EWORKSPACE;
    const size_t xb = xpass ? (size_t)M * K * 2 : 0, yb = products ? (size_t)M * N * 2 : 0,
                 qb = products ? (size_t)N * K : 0, sb = products ? (size_t)N * (size_t)(K / group) * 4 : 0;
    if (overlap(workspace, L.total, X, xb) || overlap(workspace, L.total, Wq, qb) ||
        overlap(workspace, L.total, w_scale, sb) || overlap(workspace, L.total, Y, yb) || overlap(Y, yb, X, xb) ||
        overlap(Y, yb, Wq, qb) || overlap(Y, yb, w_scale, sb))
        return LLMINT8_EINVAL;
    int8_t* ws = (int8_t*)workspace;
    int8_t* Xq = ws + L.xq;
    float* s_x = (float*)(ws + L.s_x);
    float* rg = (float*)(ws + L.rg);
    hipError_t e = hipSuccess;
    const bool small = products && N > 0 && group_small_batch(M, K, N, group);
    log_call(xpass ? (products ? "int8_matmul_group" : "int8_matmul_group_prepare") : "int8_matmul_group_products", M, K,
             N, dtype, NAN, small ? "group_small_batch" : "group_tiled");
    int8_t* Xqb = L.blocked ? ws + L.xqb : nullptr;
    if (xpass) e = stage("group_xpass", [&] { return launch_group_xpass(dtype, X, M, K, group, Xq, s_x, rg, Xqb, st); });
    if (e == hipSuccess && products && N > 0)
        e = small ? stage("gemm_group_small", [&] { return launch_gemm_group_small(dtype, Xq, Xqb, rg, Wq, w_scale, M, N, K, group, Y, st); })
                  : stage("gemm_group", [&] { return launch_gemm_group(dtype, Xq, rg, Wq, w_scale, M, N, K, group, Y, st); });
    return hip_status(e);
}

}  // namespace

LLMINT8_API int int8_matmul_group_small_batch(int64_t M, int64_t K, int64_t N, int64_t group) {
    int rc = check_group(M, K, N, LLMINT8_F16, group);
    if (rc) return rc;
    return K > 0 && N > 0 && group_small_batch(M, K, N, group) ? 1 : 0;
}

LLMINT8_API int int8_matmul_group(const void* X, int64_t M, int64_t K, int dtype, int64_t group, const int8_t* Wq,
                                  const float* w_scale, int64_t N, void* Y, void* workspace, size_t workspace_bytes,
                                  void* stream) {
    int rc = check_group(M, K, N, dtype, group);
    if (rc || M == 0 || N == 0) return rc;
    return group_common(X, M, K, dtype, group, Wq, w_scale, N, Y, workspace, workspace_bytes, stream, true, true);
}

LLMINT8_API int int8_matmul_group_prepare(const void* X, int64_t M, int64_t K, int dtype, int64_t group,
                                          void* workspace, size_t workspace_bytes, void* stream) {
    return group_common(X, M, K, dtype, group, nullptr, nullptr, 0, nullptr, workspace, workspace_bytes, stream, true,
                        false);
}

LLMINT8_API int int8_matmul_group_products(int64_t M, int64_t K, int dtype, int64_t group, const int8_t* Wq,
                                           const float* w_scale, int64_t N, void* Y, void* workspace,
                                           size_t workspace_bytes, void* stream) {
    return group_common(nullptr, M, K, dtype, group, Wq, w_scale, N, Y, workspace, workspace_bytes, stream, false,
                        true);
}

// ---- int8_matmul without a caller workspace: the same kernels on a scratch array the
// library keeps in device memory.  In host code `scratch` names a host-side stand-in, not
// the device array: its device address is looked up per device (hipGetSymbolAddress, with
// that device current) and only that address is handed to kernels.

static __device__ __align__(256) int8_t scratch[LLMINT8_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mutex;
// Stands for the scratch address where nothing may dereference it: the argument checks, and
// dry runs (LLMINT8_FAULT), which enqueue nothing.
void* const kScratchStandIn = (void*)((uintptr_t)1 << 40);

// The current device's copy of `scratch` (looked up on the first call on that device).
hipError_t scratch_for_current_device(void** out) {
    if (fault_stage()) {
        *out = kScratchStandIn;
        return stage("scratch_symbol", [] { return hipSuccess; });
    }
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        p = g_scratch[dev].load(std::memory_order_acquire);
        if (!p) {
            e = stage("scratch_symbol", [&] { return hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)); });
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

}  // namespace

LLMINT8_API int int8_matmul_noalloc(const void* X, int64_t M, int64_t K, int dtype, const int8_t* Wq,
                                    const float* w_scale, int64_t N, float threshold, void* Y, void* stream) {
    if (!Y && M > 0 && N > 0) return LLMINT8_EINVAL;
    // every argument check of int8_matmul (sizes beyond the scratch: LLMINT8_EWORKSPACE) before any HIP call
    int rc = matmul_common(X, M, K, dtype, Wq, w_scale, N, threshold, Y, nullptr, nullptr, kScratchStandIn,
                           LLMINT8_NOALLOC_SCRATCH_BYTES, stream, false);
    if (rc || M == 0) return rc;
    void* ws = nullptr;
    hipError_t e = scratch_for_current_device(&ws);
    if (e != hipSuccess) return hip_status(e);
    log_call("int8_matmul_noalloc", M, K, N, dtype, threshold, "library scratch");
    return matmul_common(X, M, K, dtype, Wq, w_scale, N, threshold, Y, nullptr, nullptr, ws,
                         LLMINT8_NOALLOC_SCRATCH_BYTES, stream);
}
