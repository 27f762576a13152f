/*
 * oracle_softmax.c -- plain FP64 row-softmax oracle (C99 + OpenMP over rows), with
 * the softmax backward and the fused residual RMSNorm on the same row layout.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the bench's
 * CPU-baseline leg load this library. The GPU product path never calls it, and
 * it shares no code, header, table or constant with the GPU library.
 *
 * What it computes, per row i of an M x N matrix stored row-major with a row
 * stride in elements (column stride 1):
 *
 *   y[i,j] = exp(x[i,j] - m_i) / sum_k exp(x[i,k] - m_i),  m_i = max_k x[i,k]
 *
 * This is the softmax the pages define in words: subtract the row maximum,
 * exponentiate, divide by the sum ("Triton: Writing GPU Kernels in Python,
 * Measured", section "Step 2: a fused softmax"; "Fused Softmax on GPU",
 * sections "The Bandwidth Formula" and "Triton -- One Block Per Row", whose
 * row-stride arguments this API keeps).  The reference value is computed in
 * FP64 and rounded once to the storage dtype (Warpline README, the paragraph
 * on how the K2 reference is formed: FP64, then one cast).
 *
 * Steps, in the order the definition states them:
 *   1. decode every stored element exactly to double (FP32 widen; FP16 and
 *      BF16 by their IEEE bit layouts);
 *   2. m = max over the row (NaN entries do not win the max; they poison the
 *      sum in step 4, so a row holding NaN comes out all NaN);
 *   3. e_j = exp(x_j - m) with libm exp in double;
 *   4. s = sum of e_j, added left to right in double;
 *   5. y_j = e_j / s in double.
 *
 * The backward of the same operation ("Measured optimization case studies",
 * section "Training: backward kernels through autograd": the softmax keeps its
 * output y and forms y * (dy - sum(y * dy))) is computed from the stored y and
 * dy, decoded exactly, by the same plain steps in FP64:
 *   1. d = sum_j y_j * dy_j, added left to right;
 *   2. dx_j = y_j * (dy_j - d).
 *
 * The fused residual RMSNorm (Warpline README, the description of its K1 kernel:
 * the input and the residual are added in FP32, that sum is rounded once to the
 * input dtype, the RMS reduction runs in FP32, the weight is applied and the result
 * is written in the input dtype), per row, from the stored x, residual r and
 * weight w:
 *   1. s_j = x_j + r_j rounded once to the dtype. The pages add in FP32 and then
 *      round; for FP16 and BF16 that equals the correctly rounded sum, because FP32
 *      carries at least 2p + 1 bits for p-bit formats (Figueroa's theorem on
 *      innocuous double rounding), and for FP32 data the double sum rounded to FP32
 *      is the FP32 sum for the same reason (53 >= 2 * 24 + 1). So the oracle adds in
 *      double and rounds once with its own encoder. No residual: s = x.
 *   2. q = sum_j s_j^2 in double, left to right;
 *   3. y_j = s_j * w_j / sqrt(q / N + eps) in double (eps is the caller's; the
 *      pages give no value).
 *
 * Scaled dot-product attention with the online softmax's result ("Fused Softmax on
 * GPU", its closing section: fusing the softmax with the matmul before it is what
 * FlashAttention does; the attention-logit workload of the same pages), per (head,
 * query) row i, from stored q, k, v, in FP64:
 *   1. S_j = scale * sum_d q_id k_jd for every key j; with the causal mask, keys
 *      j > i + (Sk - Sq) are -inf (the last query sees every key);
 *   2. P = softmax(S) exactly as above (an all -inf row gives zeros);
 *   3. O_id = sum_j P_j v_jd; lse_i = m + log(s) (-inf for an all -inf row).
 *
 * Readings where the pages are silent:
 *   - a row whose entries are all -inf (and an empty row) has no finite
 *     maximum; the online-merge guard of "Measured optimization case studies",
 *     section "Wide rows: loop in one program, or split across programs",
 *     treats such a part as shift 0 with sum 0.  For a whole row this oracle
 *     returns all zeros (masked entries give 0, and nothing is unmasked);
 *   - +inf anywhere makes exp(inf - inf) = NaN, so the row is all NaN (plain
 *     IEEE evaluation of the definition, no special case);
 *   - the final cast rounds to nearest, ties to even (IEEE default).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* dtype codes of this oracle's own API */
enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2 };

static int elem_size(int dtype) {
    switch (dtype) {
    case ORC_F32: return 4;
    case ORC_F16: return 2;
    case ORC_BF16: return 2;
    default: return 0;
    }
}

/* ---------------------------------------------------------------- decode */

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double decode_f16(uint16_t h) {
    int sign = (h >> 15) & 1;
    int ex = (h >> 10) & 0x1f;
    int fr = h & 0x3ff;
    double v;
    if (ex == 0) {
        v = ldexp((double)fr, -24); /* zero or subnormal: fr * 2^-24 */
    } else if (ex == 31) {
        v = fr ? NAN : INFINITY;
    } else {
        v = ldexp((double)(fr + 1024), ex - 25); /* 1.fr * 2^(ex-15) */
    }
    return sign ? -v : v;
}

/* bfloat16 is the upper half of an IEEE binary32. */
static double decode_bf16(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

static double decode_f32(uint32_t u) {
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

static double load_elem(const unsigned char *p, int dtype) {
    if (dtype == ORC_F32) {
        uint32_t u;
        memcpy(&u, p, 4);
        return decode_f32(u);
    }
    uint16_t h;
    memcpy(&h, p, 2);
    return dtype == ORC_F16 ? decode_f16(h) : decode_bf16(h);
}

/* ---------------------------------------------------------------- encode */

/*
 * Round a double to a binary format with `mant` stored fraction bits and an
 * exponent field of `ebits` bits, nearest-even, in one step from the double
 * (no intermediate rounding).  Returns the bit pattern.
 *
 * Method: take E = floor(log2 |v|) clamped below at the format's smallest
 * normal exponent; scale |v| by 2^(mant - E) so that one unit in the last
 * place of the target is 1.0 (a power-of-two scaling, exact in double); round
 * that to an integer with nearbyint (ties to even in the default rounding
 * mode); rebuild the fields, carrying into the exponent when the rounding
 * reaches 2^(mant+1), and overflowing to infinity above the largest exponent.
 */
static uint32_t encode_binary(double v, int mant, int ebits) {
    const int bias = (1 << (ebits - 1)) - 1;
    const int emin = 1 - bias, emax = bias;
    const uint32_t sign = signbit(v) ? (1u << (mant + ebits)) : 0u;
    const uint32_t exp_all = ((1u << ebits) - 1u) << mant;
    if (isnan(v)) return sign | exp_all | (1u << (mant - 1));
    double a = fabs(v);
    if (isinf(a)) return sign | exp_all;
    if (a == 0.0) return sign;
    int E = ilogb(a);
    if (E < emin) E = emin;
    double r = nearbyint(ldexp(a, mant - E));
    if (r >= ldexp(1.0, mant + 1)) { /* rounded up to the next binade */
        r = ldexp(1.0, mant);
        E += 1;
    }
    if (E > emax) return sign | exp_all; /* overflow to infinity */
    uint32_t q = (uint32_t)r;
    if (q < (1u << mant)) return sign | q; /* subnormal (E == emin) */
    return sign | ((uint32_t)(E + bias) << mant) | (q - (1u << mant));
}

/* ---------------------------------------------------------------- API */

int oracle_elem_size(int dtype) { return elem_size(dtype); }

int oracle_decode(const void *src, int dtype, int64_t count, double *dst) {
    int es = elem_size(dtype);
    if (!es || count < 0) return -1;
    const unsigned char *p = (const unsigned char *)src;
    for (int64_t k = 0; k < count; ++k) dst[k] = load_elem(p + k * es, dtype);
    return 0;
}

int oracle_encode(const double *src, int dtype, int64_t count, void *dst) {
    if (!elem_size(dtype) || count < 0) return -1;
    for (int64_t k = 0; k < count; ++k) {
        if (dtype == ORC_F32) {
            uint32_t u = encode_binary(src[k], 23, 8);
            memcpy((unsigned char *)dst + 4 * k, &u, 4);
        } else {
            uint16_t h = (uint16_t)(dtype == ORC_F16 ? encode_binary(src[k], 10, 5)
                                                     : encode_binary(src[k], 7, 8));
            memcpy((unsigned char *)dst + 2 * k, &h, 2);
        }
    }
    return 0;
}

/* Softmax of one decoded row x[0..n) into y[0..n). */
static void softmax_row(const double *x, int64_t n, double *y) {
    double m = -INFINITY;
    for (int64_t j = 0; j < n; ++j)
        if (x[j] > m) m = x[j];
    if (m == -INFINITY) { /* all entries -inf (or NaN-free empty row): zeros */
        int has_nan = 0;
        for (int64_t j = 0; j < n; ++j) has_nan |= isnan(x[j]);
        for (int64_t j = 0; j < n; ++j) y[j] = has_nan ? NAN : 0.0;
        return;
    }
    double s = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        y[j] = exp(x[j] - m);
        s += y[j];
    }
    for (int64_t j = 0; j < n; ++j) y[j] = y[j] / s;
}

/*
 * Softmax of selected rows.
 *   in        : base of the stored matrix (row r starts at in + r*in_stride elements)
 *   rows      : row indices to evaluate, or NULL for rows 0..nrows-1
 *   y         : output, nrows x cols doubles, contiguous
 *   threads   : OpenMP threads (<= 0: the runtime default)
 * Returns 0, or -1 on a bad argument.
 */
int oracle_softmax_rows(const void *in, int dtype, int64_t cols, int64_t in_stride,
                        const int64_t *rows, int64_t nrows, double *y, int threads) {
    int es = elem_size(dtype);
    if (!es || cols < 0 || nrows < 0 || in_stride < cols) return -1;
    if (nrows == 0 || cols == 0) return 0;
    const unsigned char *base = (const unsigned char *)in;
#ifdef _OPENMP
    if (threads <= 0) threads = omp_get_max_threads();
#else
    threads = 1;
#endif
    int bad = 0;
#pragma omp parallel num_threads(threads) reduction(| : bad)
    {
        double *x = (double *)malloc(sizeof(double) * (size_t)cols);
        if (!x) bad = 1;
#pragma omp for schedule(static)
        for (int64_t k = 0; k < nrows; ++k) {
            if (!x) continue;
            int64_t r = rows ? rows[k] : k;
            const unsigned char *row = base + (size_t)(r * in_stride) * (size_t)es;
            for (int64_t j = 0; j < cols; ++j) x[j] = load_elem(row + (size_t)j * es, dtype);
            softmax_row(x, cols, y + (size_t)k * (size_t)cols);
        }
        free(x);
    }
    return bad ? -1 : 0;
}

/* Backward of one decoded row: dx = y * (dy - sum(y * dy)). */
static void softmax_bwd_row(const double *y, const double *dy, int64_t n, double *dx) {
    double d = 0.0;
    for (int64_t j = 0; j < n; ++j) d += y[j] * dy[j];
    for (int64_t j = 0; j < n; ++j) dx[j] = y[j] * (dy[j] - d);
}

/*
 * Softmax backward of selected rows.
 *   y, dy      : stored softmax output and upstream gradient (same dtype), row r of
 *                each at base + r * stride elements
 *   rows       : row indices, or NULL for rows 0..nrows-1
 *   dx         : output, nrows x cols doubles, contiguous
 * Returns 0, or -1 on a bad argument.
 */
int oracle_softmax_bwd_rows(const void *y, const void *dy, int dtype, int64_t cols,
                            int64_t y_stride, int64_t dy_stride, const int64_t *rows,
                            int64_t nrows, double *dx, int threads) {
    int es = elem_size(dtype);
    if (!es || cols < 0 || nrows < 0 || y_stride < cols || dy_stride < cols) return -1;
    if (nrows == 0 || cols == 0) return 0;
    const unsigned char *yb = (const unsigned char *)y;
    const unsigned char *db = (const unsigned char *)dy;
#ifdef _OPENMP
    if (threads <= 0) threads = omp_get_max_threads();
#else
    threads = 1;
#endif
    int bad = 0;
#pragma omp parallel num_threads(threads) reduction(| : bad)
    {
        double *a = (double *)malloc(sizeof(double) * 2 * (size_t)cols);
        if (!a) bad = 1;
#pragma omp for schedule(static)
        for (int64_t k = 0; k < nrows; ++k) {
            if (!a) continue;
            int64_t r = rows ? rows[k] : k;
            const unsigned char *yr = yb + (size_t)(r * y_stride) * (size_t)es;
            const unsigned char *dr = db + (size_t)(r * dy_stride) * (size_t)es;
            for (int64_t j = 0; j < cols; ++j) {
                a[j] = load_elem(yr + (size_t)j * es, dtype);
                a[cols + j] = load_elem(dr + (size_t)j * es, dtype);
            }
            softmax_bwd_row(a, a + cols, cols, dx + (size_t)k * (size_t)cols);
        }
        free(a);
    }
    return bad ? -1 : 0;
}

/* Residual RMSNorm of one decoded row: s (already rounded), w, n -> y. */
static void rmsnorm_row(const double *sv, const double *w, int64_t n, double eps, double *y) {
    double q = 0.0;
    for (int64_t j = 0; j < n; ++j) q += sv[j] * sv[j];
    const double den = sqrt(q / (double)n + eps);
    for (int64_t j = 0; j < n; ++j) y[j] = sv[j] * w[j] / den;
}

/*
 * Residual RMSNorm of selected rows.
 *   x, r      : stored input and residual (same dtype), row k at base + k * stride
 *               elements; r may be NULL (s = x)
 *   w         : stored weight, cols elements
 *   rows      : row indices, or NULL for rows 0..nrows-1
 *   y         : output, nrows x cols doubles
 *   s_out     : optional (NULL), nrows x cols doubles: the rounded sums s
 * Returns 0, or -1 on a bad argument.
 */
int oracle_rmsnorm_rows(const void *x, const void *r, const void *w, int dtype, int64_t cols,
                        int64_t x_stride, int64_t r_stride, const int64_t *rows, int64_t nrows,
                        double eps, double *y, double *s_out, int threads) {
    int es = elem_size(dtype);
    if (!es || cols < 0 || nrows < 0 || x_stride < cols || (r && r_stride < cols) || !w) return -1;
    if (nrows == 0 || cols == 0) return 0;
    const int mant = dtype == ORC_F32 ? 23 : (dtype == ORC_F16 ? 10 : 7);
    const int ebits = dtype == ORC_F16 ? 5 : 8;
    const unsigned char *xb = (const unsigned char *)x;
    const unsigned char *rb = (const unsigned char *)r;
    const unsigned char *wb = (const unsigned char *)w;
#ifdef _OPENMP
    if (threads <= 0) threads = omp_get_max_threads();
#else
    threads = 1;
#endif
    int bad = 0;
#pragma omp parallel num_threads(threads) reduction(| : bad)
    {
        double *a = (double *)malloc(sizeof(double) * 2 * (size_t)cols);
        if (!a) bad = 1;
#pragma omp for schedule(static)
        for (int64_t k = 0; k < nrows; ++k) {
            if (!a) continue;
            int64_t row = rows ? rows[k] : k;
            const unsigned char *xr = xb + (size_t)(row * x_stride) * (size_t)es;
            const unsigned char *rr = rb ? rb + (size_t)(row * r_stride) * (size_t)es : NULL;
            for (int64_t j = 0; j < cols; ++j) {
                double v = load_elem(xr + (size_t)j * es, dtype);
                if (rr) {
                    const uint32_t bits = encode_binary(v + load_elem(rr + (size_t)j * es, dtype),
                                                        mant, ebits);
                    unsigned char buf[4];
                    if (es == 4) {
                        memcpy(buf, &bits, 4);
                    } else {
                        const uint16_t h = (uint16_t)bits;
                        memcpy(buf, &h, 2);
                    }
                    v = load_elem(buf, dtype);
                }
                a[j] = v;
                a[cols + j] = load_elem(wb + (size_t)j * es, dtype);
            }
            rmsnorm_row(a, a + cols, cols, eps, y + (size_t)k * (size_t)cols);
            if (s_out) memcpy(s_out + (size_t)k * (size_t)cols, a, sizeof(double) * (size_t)cols);
        }
        free(a);
    }
    return bad ? -1 : 0;
}

/*
 * Attention of selected rows.
 *   q, k, v   : stored [BH][S][d] tensors (same dtype), element (h, i, c) at
 *               base + h * head_stride + i * row_stride + c
 *   rows      : flat row indices h * Sq + i, or NULL for all BH * Sq rows
 *   o         : output, nrows x d doubles; lse: nrows doubles (may be NULL)
 * Returns 0, or -1 on a bad argument.
 */
int oracle_attention_rows(const void *q, const void *k, const void *v, int dtype, int64_t BH,
                          int64_t Sq, int64_t Sk, int64_t d, int64_t q_rs, int64_t q_hs,
                          int64_t k_rs, int64_t k_hs, int64_t v_rs, int64_t v_hs, double scale,
                          int causal, const int64_t *rows, int64_t nrows, double *o, double *lse,
                          int threads) {
    int es = elem_size(dtype);
    if (!es || BH < 0 || Sq < 0 || Sk < 0 || d <= 0 || nrows < 0) return -1;
    if (nrows == 0) return 0;
    const unsigned char *qb = (const unsigned char *)q;
    const unsigned char *kb = (const unsigned char *)k;
    const unsigned char *vb = (const unsigned char *)v;
#ifdef _OPENMP
    if (threads <= 0) threads = omp_get_max_threads();
#else
    threads = 1;
#endif
    int bad = 0;
#pragma omp parallel num_threads(threads) reduction(| : bad)
    {
        double *buf = (double *)malloc(sizeof(double) * (size_t)(d + 2 * (Sk > 0 ? Sk : 1)));
        if (!buf) bad = 1;
#pragma omp for schedule(static)
        for (int64_t t = 0; t < nrows; ++t) {
            if (!buf) continue;
            const int64_t r = rows ? rows[t] : t;
            if (r < 0 || r >= BH * Sq) {
                bad = 1;
                continue;
            }
            const int64_t h = r / Sq, i = r % Sq;
            double *qi = buf, *sv = buf + d, *pv = buf + d + Sk;
            for (int64_t c = 0; c < d; ++c)
                qi[c] = load_elem(qb + (size_t)(h * q_hs + i * q_rs + c) * es, dtype);
            for (int64_t j = 0; j < Sk; ++j) {
                if (causal && j > i + (Sk - Sq)) {
                    sv[j] = -INFINITY;
                    continue;
                }
                double acc = 0.0;
                for (int64_t c = 0; c < d; ++c)
                    acc += qi[c] * load_elem(kb + (size_t)(h * k_hs + j * k_rs + c) * es, dtype);
                sv[j] = scale * acc;
            }
            double m = -INFINITY;
            for (int64_t j = 0; j < Sk; ++j)
                if (sv[j] > m) m = sv[j];
            softmax_row(sv, Sk, pv);
            double *oi = o + (size_t)t * (size_t)d;
            for (int64_t c = 0; c < d; ++c) oi[c] = 0.0;
            for (int64_t j = 0; j < Sk; ++j) {
                if (sv[j] == -INFINITY) continue; /* masked keys do not take part */
                for (int64_t c = 0; c < d; ++c)
                    oi[c] += pv[j] * load_elem(vb + (size_t)(h * v_hs + j * v_rs + c) * es, dtype);
            }
            if (lse) {
                if (m == -INFINITY) {
                    lse[t] = -INFINITY;
                } else {
                    double ssum = 0.0;
                    for (int64_t j = 0; j < Sk; ++j) ssum += exp(sv[j] - m);
                    lse[t] = m + log(ssum);
                }
            }
        }
        free(buf);
    }
    return bad ? -1 : 0;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
