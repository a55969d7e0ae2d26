/*
 * CPU oracle for the LLM.int8() matrix multiply -- TEST INFRASTRUCTURE ONLY.
 * See oracle.h for what is computed, the readings taken, and who may use it.
 *
 * Build: gcc -std=c11 -O2 -ffp-contract=off -fopenmp -fPIC -shared (no -ffast-math,
 * no -mfma: every float op below rounds once, in the order written).
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int g_threads = 0;

int orc_set_threads(int n) {
#ifdef _OPENMP
    g_threads = n > 0 ? n : omp_get_num_procs();
#else
    (void)n;
    g_threads = 1;
#endif
    return g_threads;
}

static int nthreads(void) {
    if (g_threads <= 0) orc_set_threads(0);
    return g_threads;
}

/* ------------------------------------------------------------------ formats */

static float bits_to_float(uint32_t u) {
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static uint32_t float_to_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return u;
}

/* IEEE binary16 -> binary32, exact. */
static float f16_to_f32(uint16_t h) {
    uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
    uint32_t e = (h >> 10) & 0x1fu, m = h & 0x3ffu;
    if (e == 0) {
        float v = (float)m * 0x1p-24f; /* subnormal: m * 2^-24, exact */
        return sign ? -v : v;
    }
    if (e == 31) return bits_to_float(sign | 0x7f800000u | (m << 13));
    return bits_to_float(sign | ((e + 112u) << 23) | (m << 13));
}

/* binary32 -> binary16, round to nearest even; overflow -> inf; NaN stays NaN. */
static uint16_t f32_to_f16(float f) {
    uint32_t x = float_to_bits(f);
    uint16_t sign = (uint16_t)((x >> 16) & 0x8000u);
    uint32_t ax = x & 0x7fffffffu;
    if (ax > 0x7f800000u) return (uint16_t)(sign | 0x7e00u | ((ax >> 13) & 0x3ffu));
    if (ax >= 0x477ff000u) return (uint16_t)(sign | 0x7c00u); /* >= 65520 rounds to inf */
    if (ax < 0x38800000u) {                                 /* below 2^-14: fp16 subnormal or 0 */
        float m = rintf(bits_to_float(ax) * 0x1p24f);       /* scaling by 2^24 is exact */
        return (uint16_t)(sign | (uint16_t)m);
    }
    uint32_t r = ax - 0x38000000u; /* rebias the exponent from 127 to 15 */
    r += 0xfffu + ((r >> 13) & 1u);
    return (uint16_t)(sign | (uint16_t)(r >> 13));
}

static float bf16_to_f32(uint16_t h) { return bits_to_float((uint32_t)h << 16); }

static uint16_t f32_to_bf16(float f) {
    uint32_t x = float_to_bits(f);
    if ((x & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((x >> 16) | 0x40u);
    x += 0x7fffu + ((x >> 16) & 1u);
    return (uint16_t)(x >> 16);
}

float orc_to_f32(uint16_t h, int dt) { return dt == ORC_BF16 ? bf16_to_f32(h) : f16_to_f32(h); }

uint16_t orc_from_f32(float f, int dt) { return dt == ORC_BF16 ? f32_to_bf16(f) : f32_to_f16(f); }

void orc_to_f32_n(const uint16_t* h, int64_t n, int dt, float* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_to_f32(h[i], dt);
}

void orc_from_f32_n(const float* f, int64_t n, int dt, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_from_f32(f[i], dt);
}

/* ---------------------------------------------------------------- quantizer */

/* One normalization constant per vector: the vector's absmax s maps to 127. */
float orc_inv_scale(float s) { return s > 0.0f ? 127.0f / s : 0.0f; }

/* Round to nearest (ties to even), then keep the symmetric range [-127, 127]. */
int8_t orc_quantize(float x, float inv) {
    float v = rintf(x * inv);
    if (v > 127.0f) v = 127.0f;
    if (v < -127.0f) v = -127.0f;
    return (int8_t)v;
}

void orc_quantize_n(const float* x, int64_t n, float s, int8_t* q) {
    float inv = orc_inv_scale(s);
    for (int64_t i = 0; i < n; ++i) q[i] = orc_quantize(x[i], inv);
}

/* ------------------------------------------------------ weight (offline) */

void orc_quantize_weight(const uint16_t* W, int64_t K, int64_t N, int dt, int8_t* Wq, float* s_w) {
    /* Columns are handled in blocks of 64 so that each row of W is read contiguously;
     * every column still gets exactly the max and the quantizer of its own values. */
    int nt = nthreads();
#pragma omp parallel for num_threads(nt) schedule(static)
    for (int64_t nb = 0; nb < N; nb += 64) {
        int64_t ne = nb + 64 < N ? nb + 64 : N;
        float s[64], inv[64];
        for (int64_t n = nb; n < ne; ++n) s[n - nb] = 0.0f;
        for (int64_t k = 0; k < K; ++k)
            for (int64_t n = nb; n < ne; ++n) {
                float a = fabsf(orc_to_f32(W[k * N + n], dt));
                if (a > s[n - nb]) s[n - nb] = a;
            }
        for (int64_t n = nb; n < ne; ++n) {
            s_w[n] = s[n - nb];
            inv[n - nb] = orc_inv_scale(s[n - nb]);
        }
        for (int64_t k = 0; k < K; ++k)
            for (int64_t n = nb; n < ne; ++n)
                Wq[n * K + k] = orc_quantize(orc_to_f32(W[k * N + n], dt), inv[n - nb]);
    }
}

/* ------------------------------------------------------------- X: outliers */

int64_t orc_outlier_columns(const uint16_t* X, int64_t M, int64_t K, int dt, float tau, int32_t* O) {
    unsigned char* flag = (unsigned char*)calloc((size_t)(K > 0 ? K : 1), 1);
    int nt = nthreads();
    /* each thread owns a block of 64 columns and scans every row of it */
#pragma omp parallel for num_threads(nt) schedule(static)
    for (int64_t jb = 0; jb < K; jb += 64) {
        int64_t je = jb + 64 < K ? jb + 64 : K;
        for (int64_t i = 0; i < M; ++i)
            for (int64_t j = jb; j < je; ++j)
                if (fabsf(orc_to_f32(X[i * K + j], dt)) > tau) flag[j] = 1;
    }
    int64_t n = 0;
    for (int64_t j = 0; j < K; ++j)
        if (flag[j]) O[n++] = (int32_t)j;
    free(flag);
    return n;
}

/* ------------------------------------------------------- X: quantize rows */

void orc_quantize_rows(const uint16_t* X, int64_t M, int64_t K, int dt, const int32_t* O, int64_t nO,
                       int8_t* Xq, float* s_x, uint16_t* XO) {
    unsigned char* is_out = (unsigned char*)calloc((size_t)(K > 0 ? K : 1), 1);
    for (int64_t t = 0; t < nO; ++t) is_out[O[t]] = 1;
    int nt = nthreads();
#pragma omp parallel for num_threads(nt) schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        const uint16_t* row = X + i * K;
        float s = 0.0f;
        for (int64_t j = 0; j < K; ++j) {
            if (is_out[j]) continue;
            float a = fabsf(orc_to_f32(row[j], dt));
            if (a > s) s = a;
        }
        s_x[i] = s;
        float inv = orc_inv_scale(s);
        for (int64_t j = 0; j < K; ++j) Xq[i * K + j] = is_out[j] ? 0 : orc_quantize(orc_to_f32(row[j], dt), inv);
        for (int64_t t = 0; t < nO; ++t) XO[i * nO + t] = row[O[t]];
    }
    free(is_out);
}

/* --------------------------------------------------------- int8 part */

int orc_int_gemm(const int8_t* Xq, const int8_t* Wq, int64_t K, int64_t N,
                 const int64_t* rows, int64_t nrows, int32_t* C) {
    int bad = 0;
    int nt = nthreads();
#pragma omp parallel for num_threads(nt) schedule(dynamic, 1) reduction(| : bad)
    for (int64_t r = 0; r < nrows; ++r) {
        const int8_t* x = Xq + (rows ? rows[r] : r) * K;
        for (int64_t n = 0; n < N; ++n) {
            const int8_t* w = Wq + n * K;
            int64_t acc = 0;
            for (int64_t k = 0; k < K; ++k) acc += (int64_t)x[k] * (int64_t)w[k];
            if (acc > INT32_MAX || acc < INT32_MIN) bad = 1;
            C[r * N + n] = (int32_t)acc;
        }
    }
    return bad ? -1 : 0;
}

/* ------------------------------------------------------- 16-bit part */

void orc_outlier_gemm(const uint16_t* XO, int64_t nO, int dt, const int8_t* Wq, int64_t K, int64_t N,
                      const int32_t* O, const int64_t* rows, int64_t nrows,
                      float* F, double* F64, double* A) {
    int nt = nthreads();
#pragma omp parallel for num_threads(nt) schedule(static)
    for (int64_t r = 0; r < nrows; ++r) {
        const uint16_t* xo = XO + (rows ? rows[r] : r) * nO;
        for (int64_t n = 0; n < N; ++n) {
            float f = 0.0f;
            double f64 = 0.0, a = 0.0;
            for (int64_t t = 0; t < nO; ++t) {
                float xv = orc_to_f32(xo[t], dt);
                float wv = (float)Wq[n * K + O[t]]; /* exact in either 16-bit type */
                float p = xv * wv;                  /* exact: <= 11 x 7 significant bits */
                f = f + p;
                f64 += (double)p;
                a += fabs((double)p);
            }
            F[r * N + n] = f;
            if (F64) F64[r * N + n] = f64;
            if (A) A[r * N + n] = a;
        }
    }
}

/* ----------------------------------------------------------- epilogue */

void orc_dequant(const int32_t* C, const float* F, const float* s_x_rows, const float* s_w,
                 int64_t nrows, int64_t N, int dt, float* y, uint16_t* Y) {
    for (int64_t r = 0; r < nrows; ++r) {
        float ri = s_x_rows[r] / 127.0f;
        for (int64_t n = 0; n < N; ++n) {
            float cn = s_w[n] / 127.0f;
            float cf = (float)C[r * N + n];
            float yi = (cf * ri) * cn;
            float yo = cn * F[r * N + n];
            float v = yi + yo;
            if (y) y[r * N + n] = v;
            Y[r * N + n] = orc_from_f32(v, dt);
        }
    }
}

/* ------------------------------------------------ fixed outlier dimensions */

void orc_quantize_weight_fixed(const uint16_t* W, int64_t K, int64_t N, int dt, const int32_t* O, int64_t nO,
                               int8_t* Wq, float* s_w, uint16_t* WO) {
    unsigned char* is_out = (unsigned char*)calloc((size_t)(K > 0 ? K : 1), 1);
    for (int64_t t = 0; t < nO; ++t) is_out[O[t]] = 1;
    int nt = nthreads();
#pragma omp parallel for num_threads(nt) schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        float s = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            if (is_out[k]) continue;
            float a = fabsf(orc_to_f32(W[k * N + n], dt));
            if (a > s) s = a;
        }
        s_w[n] = s;
        float inv = orc_inv_scale(s);
        for (int64_t k = 0; k < K; ++k)
            Wq[n * K + k] = is_out[k] ? 0 : orc_quantize(orc_to_f32(W[k * N + n], dt), inv);
        for (int64_t t = 0; t < nO; ++t) WO[n * nO + t] = W[(int64_t)O[t] * N + n];
    }
    free(is_out);
}

void orc_outlier_gemm_exact(const uint16_t* XO, int64_t nO, int dt, const uint16_t* WO, int64_t N,
                            const int64_t* rows, int64_t nrows, float* F, double* F64, double* A) {
    int nt = nthreads();
#pragma omp parallel for num_threads(nt) schedule(static)
    for (int64_t r = 0; r < nrows; ++r) {
        const uint16_t* xo = XO + (rows ? rows[r] : r) * nO;
        for (int64_t n = 0; n < N; ++n) {
            float sum = 0.0f;
            double sum64 = 0.0, mag = 0.0;
            for (int64_t t = 0; t < nO; ++t) {
                float prod = orc_to_f32(xo[t], dt) * orc_to_f32(WO[n * nO + t], dt); /* exact: <= 22 bits */
                sum = sum + prod;
                sum64 += (double)prod;
                mag += fabs((double)prod);
            }
            F[r * N + n] = sum;
            if (F64) F64[r * N + n] = sum64;
            if (A) A[r * N + n] = mag;
        }
    }
}

void orc_dequant_fixed(const int32_t* C, const float* F, const float* s_x_rows, const float* s_w,
                       int64_t nrows, int64_t N, int dt, float* y, uint16_t* Y) {
    for (int64_t r = 0; r < nrows; ++r) {
        float ri = s_x_rows[r] / 127.0f;
        for (int64_t n = 0; n < N; ++n) {
            float cn = s_w[n] / 127.0f;
            float cf = (float)C[r * N + n];
            float y_int = (cf * ri) * cn;
            float v = y_int + F[r * N + n];
            if (y) y[r * N + n] = v;
            Y[r * N + n] = orc_from_f32(v, dt);
        }
    }
}

/* ------------------------------------------------------ group-wise scales */

void orc_group_quantize_rows(const uint16_t* X, int64_t M, int64_t K, int dt, int64_t G, int8_t* Xq, float* s_x) {
    int64_t ng = K / G;
    int nt = nthreads();
#pragma omp parallel for num_threads(nt) schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t g = 0; g < ng; ++g) {
            const uint16_t* xs = X + i * K + g * G;
            float s = 0.0f;
            for (int64_t k = 0; k < G; ++k) {
                float a = fabsf(orc_to_f32(xs[k], dt));
                if (a > s) s = a;
            }
            s_x[i * ng + g] = s;
            float inv = orc_inv_scale(s);
            for (int64_t k = 0; k < G; ++k) Xq[i * K + g * G + k] = orc_quantize(orc_to_f32(xs[k], dt), inv);
        }
    }
}

void orc_group_quantize_weight(const uint16_t* W, int64_t K, int64_t N, int dt, int64_t G, int8_t* Wq, float* s_w) {
    int64_t ng = K / G;
    int nt = nthreads();
#pragma omp parallel for num_threads(nt) schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t g = 0; g < ng; ++g) {
            float s = 0.0f;
            for (int64_t k = g * G; k < (g + 1) * G; ++k) {
                float a = fabsf(orc_to_f32(W[k * N + n], dt));
                if (a > s) s = a;
            }
            s_w[n * ng + g] = s;
            float inv = orc_inv_scale(s);
            for (int64_t k = g * G; k < (g + 1) * G; ++k) Wq[n * K + k] = orc_quantize(orc_to_f32(W[k * N + n], dt), inv);
        }
    }
}

void orc_group_gemm(const int8_t* Xq, const float* s_x, const int8_t* Wq, const float* s_w, int64_t K, int64_t N,
                    int64_t G, const int64_t* rows, int64_t nrows, int dt, float* y, uint16_t* Y) {
    int64_t ng = K / G;
    int nt = nthreads();
#pragma omp parallel for num_threads(nt) schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t i = rows ? rows[r] : r;
        const int8_t* x = Xq + i * K;
        for (int64_t n = 0; n < N; ++n) {
            const int8_t* wrow = Wq + n * K;
            float acc = 0.0f;
            for (int64_t g = 0; g < ng; ++g) {
                int32_t cg = 0;
                for (int64_t k = g * G; k < (g + 1) * G; ++k) cg += (int32_t)x[k] * (int32_t)wrow[k];
                float rg = s_x[i * ng + g] / 127.0f;
                float cng = s_w[n * ng + g] / 127.0f;
                float term = ((float)cg * rg) * cng;
                acc = acc + term;
            }
            if (y) y[r * N + n] = acc;
            Y[r * N + n] = orc_from_f32(acc, dt);
        }
    }
}

/* ------------------------------------------------------- block-wise codec */

void orc_block_quantize(const float* x, int64_t n, int64_t block, int8_t* q, float* absmax) {
    int64_t nb = (n + block - 1) / block;
    int nt = nthreads();
#pragma omp parallel for num_threads(nt) schedule(static)
    for (int64_t b = 0; b < nb; ++b) {
        int64_t lo = b * block, hi = lo + block < n ? lo + block : n;
        float s = 0.0f;
        for (int64_t i = lo; i < hi; ++i) {
            float a = fabsf(x[i]);
            if (a > s) s = a;
        }
        absmax[b] = s;
        float inv = orc_inv_scale(s);
        for (int64_t i = lo; i < hi; ++i) q[i] = orc_quantize(x[i], inv);
    }
}

void orc_block_dequantize(const int8_t* q, const float* absmax, int64_t n, int64_t block, float* x) {
    int64_t nb = (n + block - 1) / block;
    int nt = nthreads();
#pragma omp parallel for num_threads(nt) schedule(static)
    for (int64_t b = 0; b < nb; ++b) {
        int64_t lo = b * block, hi = lo + block < n ? lo + block : n;
        float step = absmax[b] / 127.0f;
        for (int64_t i = lo; i < hi; ++i) x[i] = (float)q[i] * step;
    }
}
