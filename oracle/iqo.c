/*
 * iqo.c -- plain, slow CPU oracle for integer-quantized convolution and GEMM.
 *
 * TEST INFRASTRUCTURE ONLY: the byte-exact reference the GPU library is checked
 * against.  It is loaded by the tests, the smoke check and the benchmark's
 * CPU-baseline leg, never by the product path, and it shares no code with the
 * GPU library.
 *
 * Each function writes out the plain definition: direct loops, explicit
 * (q - Z) subtraction instead of any zero-point folding, int64 accumulation,
 * one IEEE binary32 rounding per floating-point operation.  Built with
 * -ffp-contract=off -fno-fast-math so no multiply-add is fused and nothing is
 * reassociated.  The only parallelism is OpenMP over independent output rows;
 * integer sums are exact, so their order does not matter.
 *
 * Page citations: see iqo.h for the page list.  Readings of points the pages
 * leave open are marked "READING".
 */
#include "iqo.h"

#include <fenv.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int iqo_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads of the OpenMP loops that follow (n >= 1); for timing the oracle on one core
 * and on all of them.  Results do not depend on it (integer sums are exact). */
void iqo_set_num_threads(int n) {
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Code ranges.
 * "Quantization" blog, section 量化模式 (quantization modes): symmetric mode clips
 * to int8, asymmetric mode to uint8; section 量化参数选择 notes that int8 really
 * reaches -128.  MegEngine 4-bit article, Fig. 1 / Fig. 2: UINT4 is [0, 15],
 * INT4 is [-8, 7]. */
int iqo_qrange(int qtype, int32_t *qmin, int32_t *qmax) {
    switch (qtype) {
    case IQO_INT8:  *qmin = -128; *qmax = 127; return IQO_OK;
    case IQO_UINT8: *qmin = 0;    *qmax = 255; return IQO_OK;
    case IQO_INT4:  *qmin = -8;   *qmax = 7;   return IQO_OK;
    case IQO_UINT4: *qmin = 0;    *qmax = 15;  return IQO_OK;
    case IQO_INT32: *qmin = INT32_MIN; *qmax = INT32_MAX; return IQO_OK;
    default: return IQO_EINVAL;
    }
}

/* Round to the nearest integer, ties to even.
 * "Quantization" blog, section 量化算子: the round function's tie mode differs
 * between hardware; torch and C use round-half-to-even.  nearbyintf in the
 * default FE_TONEAREST mode is exactly that (roundf would round ties away). */
static float rne(float v) { return nearbyintf(v); }

/* Clamp a rounded float into a range where the float->int conversion is
 * defined; every clip range used here lies well inside +-2^30. */
static int64_t f2i_sat(float r) {
    if (r > 1073741824.0f) r = 1073741824.0f;
    if (r < -1073741824.0f) r = -1073741824.0f;
    return (int64_t)r;
}

static int32_t clip64(int64_t v, int32_t lo, int32_t hi) {
    if (v < lo) return lo;
    if (v > hi) return hi;
    return (int32_t)v;
}

static int scale_ok(float s) { return isfinite(s) && s > 0.0f; }

/* Quantize.
 * "Quantization" blog, section 量化算子 (basic formula): qt_32 = round_fn(value /
 * scale), then qt_8 = clip(qt_32, Q_MIN, Q_MAX); section 量化模式 (asymmetric):
 * the offset is added to the rounded quotient before the clip.  Section
 * tensor量化与通道量化: scale and offset per tensor or per channel.
 * READING: the quotient is one correctly rounded binary32 division (not a
 * multiply by 1/S); the integer zero-point is added after rounding. */
int iqo_quantize(const float *x, int32_t *q, int64_t outer, int64_t ch, int64_t inner,
                 const float *scale, const int32_t *zp, int per_channel, int qtype) {
    int32_t qmin, qmax;
    if (qtype == IQO_INT32 || iqo_qrange(qtype, &qmin, &qmax) != IQO_OK) return IQO_EINVAL;
    if (outer < 0 || ch <= 0 || inner <= 0) return IQO_EINVAL;
    int64_t nsc = per_channel ? ch : 1;
    for (int64_t c = 0; c < nsc; ++c)
        if (!scale_ok(scale[c])) return IQO_EINVAL;
    if (fegetround() != FE_TONEAREST) return IQO_EINVAL;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t o = 0; o < outer; ++o) {
        for (int64_t c = 0; c < ch; ++c) {
            float s = per_channel ? scale[c] : scale[0];
            int32_t z = per_channel ? zp[c] : zp[0];
            for (int64_t i = 0; i < inner; ++i) {
                int64_t idx = (o * ch + c) * inner + i;
                float v = x[idx];
                if (isnan(v)) { bad = 1; continue; }
                float quot = v / s;                    /* value / scale */
                float rounded = rne(quot);             /* round_fn */
                int64_t qt = f2i_sat(rounded) + z;     /* + offset */
                q[idx] = clip64(qt, qmin, qmax);       /* clip to [Q_MIN, Q_MAX] */
            }
        }
    }
    return bad ? IQO_EINVAL : IQO_OK;
}

/* Dequantize.
 * "Quantization" blog, section 反量化算子: deq = value * scale (symmetric case);
 * MegEngine 4-bit article, section 背景: r = S (Q - Z).  q - Z is an exact
 * integer, so the only rounding is the one multiply. */
int iqo_dequantize(const int32_t *q, float *x, int64_t outer, int64_t ch, int64_t inner,
                   const float *scale, const int32_t *zp, int per_channel) {
    if (outer < 0 || ch <= 0 || inner <= 0) return IQO_EINVAL;
    int64_t nsc = per_channel ? ch : 1;
    for (int64_t c = 0; c < nsc; ++c)
        if (!scale_ok(scale[c])) return IQO_EINVAL;
#pragma omp parallel for schedule(static)
    for (int64_t o = 0; o < outer; ++o) {
        for (int64_t c = 0; c < ch; ++c) {
            float s = per_channel ? scale[c] : scale[0];
            int32_t z = per_channel ? zp[c] : zp[0];
            for (int64_t i = 0; i < inner; ++i) {
                int64_t idx = (o * ch + c) * inner + i;
                float centred = (float)(q[idx] - z);
                x[idx] = centred * s;
            }
        }
    }
    return IQO_OK;
}

/* Byte packing.
 * MegEngine 4-bit article, section conv 算子優化: eight 4-bit values share one
 * 32-bit word on write-back.  READING: element 2j sits in the low nibble of
 * byte j, element 2j+1 in the high nibble; INT4 is two's complement. */
int iqo_pack(const int32_t *q, uint8_t *bytes, int64_t n, int qtype) {
    int32_t qmin, qmax;
    if (qtype == IQO_INT32 || iqo_qrange(qtype, &qmin, &qmax) != IQO_OK || n < 0) return IQO_EINVAL;
    for (int64_t i = 0; i < n; ++i)
        if (q[i] < qmin || q[i] > qmax) return IQO_EINVAL;
    if (qtype == IQO_INT8 || qtype == IQO_UINT8) {
        for (int64_t i = 0; i < n; ++i) bytes[i] = (uint8_t)(q[i] & 0xFF);
        return IQO_OK;
    }
    if (n % 2) return IQO_EINVAL;
    for (int64_t j = 0; j < n / 2; ++j) {
        uint8_t lo = (uint8_t)(q[2 * j] & 0xF);
        uint8_t hi = (uint8_t)(q[2 * j + 1] & 0xF);
        bytes[j] = (uint8_t)(lo | (hi << 4));
    }
    return IQO_OK;
}

int iqo_unpack(const uint8_t *bytes, int32_t *q, int64_t n, int qtype) {
    if (n < 0) return IQO_EINVAL;
    switch (qtype) {
    case IQO_UINT8:
        for (int64_t i = 0; i < n; ++i) q[i] = bytes[i];
        return IQO_OK;
    case IQO_INT8:
        for (int64_t i = 0; i < n; ++i) q[i] = bytes[i] < 128 ? bytes[i] : (int32_t)bytes[i] - 256;
        return IQO_OK;
    case IQO_UINT4:
    case IQO_INT4:
        if (n % 2) return IQO_EINVAL;
        for (int64_t i = 0; i < n; ++i) {
            int32_t nib = (i % 2 == 0) ? (bytes[i / 2] & 0xF) : (bytes[i / 2] >> 4);
            if (qtype == IQO_INT4 && nib >= 8) nib -= 16;
            q[i] = nib;
        }
        return IQO_OK;
    default:
        return IQO_EINVAL;
    }
}

/* Requant multiplier M = S_in * S_w / S_out, computed once before inference.
 * "Quantization" blog, section 量化乘法: the combined scale scale_abc can be
 * computed in advance.  READING: two binary32 operations in this order. */
float iqo_requant_multiplier(float s_in, float s_w, float s_out) {
    float sw_in = s_in * s_w;
    return sw_in / s_out;
}

/* Residual multiplier S_res / S_out.
 * "Quantization" blog, section 量化加法 (general form with separate scales). */
float iqo_residual_multiplier(float s_res, float s_out) { return s_res / s_out; }

/* Bias in accumulator units: rne(B / (S_in * S_w)).
 * MegEngine 4-bit article, section 緩解精度下降: the terms known before inference
 * are folded into the bias.  READING: the bias is carried as an int32 in the
 * accumulator's units (the fp32-bias form on the page is not used). */
int iqo_quantize_bias(float b, float s_in, float s_w, int32_t *bias_q) {
    float sw_in = s_in * s_w;
    float quot = b / sw_in;
    float r = rne(quot);
    if (!(r >= -2147483648.0f && r <= 2147483520.0f)) return IQO_EOVERFLOW;
    *bias_q = (int32_t)r;
    return IQO_OK;
}

/* Direct convolution accumulator (no zero-point folding, no im2col).
 * MegEngine 4-bit article, section 緩解精度下降: the quantized conv is the sum of
 * Q(W) and Q(I) products with their zero points removed, plus the bias; the
 * FP32 conv it stands for is O = sum W*I + B.  "Quantization" blog, section
 * 常见计算图优化 (conv-add fusion): Y = WX + B.
 * READING: positions outside the image hold the real value 0, i.e. code z_in. */
int iqo_conv2d_acc(const int32_t *x, int n, int h, int w, int c_in, int32_t z_in,
                   const int32_t *wt, int c_out, int kh, int kw, int32_t z_w,
                   int sh, int sw, int ph, int pw, const int32_t *bias_q, int64_t *acc) {
    if (n < 0 || h <= 0 || w <= 0 || c_in <= 0 || c_out <= 0 || kh <= 0 || kw <= 0 ||
        sh <= 0 || sw <= 0 || ph < 0 || pw < 0)
        return IQO_EINVAL;
    int oh = (h + 2 * ph - kh) / sh + 1;
    int ow = (w + 2 * pw - kw) / sw + 1;
    if (h + 2 * ph < kh || w + 2 * pw < kw || oh <= 0 || ow <= 0) return IQO_EINVAL;
    int64_t rows = (int64_t)n * oh * ow;
    int ovf = 0;
#pragma omp parallel for schedule(static) reduction(| : ovf)
    for (int64_t row = 0; row < rows; ++row) {
        int ni = (int)(row / ((int64_t)oh * ow));
        int oy = (int)((row / ow) % oh);
        int ox = (int)(row % ow);
        for (int oc = 0; oc < c_out; ++oc) {
            int64_t s = bias_q ? bias_q[oc] : 0;
            for (int ky = 0; ky < kh; ++ky) {
                for (int kx = 0; kx < kw; ++kx) {
                    int iy = oy * sh - ph + ky;
                    int ix = ox * sw - pw + kx;
                    int inside = iy >= 0 && iy < h && ix >= 0 && ix < w;
                    for (int ci = 0; ci < c_in; ++ci) {
                        int32_t xv = inside ? x[(((int64_t)ni * h + iy) * w + ix) * c_in + ci] : z_in;
                        int32_t wv = wt[(((int64_t)oc * kh + ky) * kw + kx) * c_in + ci];
                        s += (int64_t)(xv - z_in) * (int64_t)(wv - z_w);
                    }
                }
            }
            if (s < INT32_MIN || s > INT32_MAX) ovf = 1;
            acc[row * c_out + oc] = s;
        }
    }
    return ovf ? IQO_EOVERFLOW : IQO_OK;
}

/* Naive GEMM accumulator.
 * "Quantization" blog, section 量化矩阵乘: int8 inputs, products in int16/32,
 * sums kept in int32/64, then requantized to int8.
 * READING: B is stored [n][k] (weight layout), so acc = (A - Z_a)(B - Z_b)^T. */
int iqo_gemm_acc(const int32_t *a, int64_t m, int64_t k, int32_t z_a, const int32_t *b,
                 int64_t n, int32_t z_b, const int32_t *bias_q, int64_t *acc) {
    if (m < 0 || k <= 0 || n <= 0) return IQO_EINVAL;
    int ovf = 0;
#pragma omp parallel for schedule(static) reduction(| : ovf)
    for (int64_t i = 0; i < m; ++i) {
        for (int64_t j = 0; j < n; ++j) {
            int64_t s = bias_q ? bias_q[j] : 0;
            for (int64_t kk = 0; kk < k; ++kk)
                s += (int64_t)(a[i * k + kk] - z_a) * (int64_t)(b[j * k + kk] - z_b);
            if (s < INT32_MIN || s > INT32_MAX) ovf = 1;
            acc[i * n + j] = s;
        }
    }
    return ovf ? IQO_EOVERFLOW : IQO_OK;
}

/* Requantizing epilogue.
 * "Quantization" blog: section 量化乘法 (rescale by the precomputed combined
 * scale, then round_fn and clip), section 量化加法 (general add
 * (a*s_a + b*s_b)/s_c), section 量化激活函数 (relu / clip are passive: same
 * scale in and out, so ReLU is a clamp at the real value 0).
 * MegEngine 4-bit article, section 算子融合優化: the fused Conv_Relu and
 * Conv_Add_Relu operators.
 * READING (fp32 evaluation order, one rounding per step):
 *   a = float(acc); t = a * M[c];
 *   ADD:  t = t + float(r - Z_res) * M_res   (two products, then the sum)
 *   RELU: t = max(t, 0)
 *   q = clip(rne(t) + Z_out, Q_MIN, Q_MAX). */
int iqo_requant(const int64_t *acc, int64_t rows, int64_t ch, const float *mult, int epi,
                const int32_t *res, int32_t z_res, float m_res, int32_t z_out, int out_qtype,
                int32_t *out) {
    int32_t qmin, qmax;
    if (rows < 0 || ch <= 0 || iqo_qrange(out_qtype, &qmin, &qmax) != IQO_OK) return IQO_EINVAL;
    if ((epi == IQO_EPI_RAW) != (out_qtype == IQO_INT32)) return IQO_EINVAL;
    if (epi < IQO_EPI_NONE || epi > IQO_EPI_RAW) return IQO_EINVAL;
    int has_add = epi == IQO_EPI_ADD || epi == IQO_EPI_ADD_RELU;
    int has_relu = epi == IQO_EPI_RELU || epi == IQO_EPI_ADD_RELU;
    if (has_add && res == NULL) return IQO_EINVAL;
    if (fegetround() != FE_TONEAREST) return IQO_EINVAL;
    int ovf = 0;
#pragma omp parallel for schedule(static) reduction(| : ovf)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t c = 0; c < ch; ++c) {
            int64_t v = acc[r * ch + c];
            if (v < INT32_MIN || v > INT32_MAX) { ovf = 1; continue; }
            if (epi == IQO_EPI_RAW) { out[r * ch + c] = (int32_t)v; continue; }
            float a = (float)(int32_t)v;     /* int32 -> binary32, nearest-even */
            float t = a * mult[c];
            if (has_add) {
                float centred = (float)(res[r * ch + c] - z_res);
                float u = centred * m_res;
                t = t + u;
            }
            if (has_relu && !(t > 0.0f)) t = 0.0f;
            float rounded = rne(t);
            out[r * ch + c] = clip64(f2i_sat(rounded) + z_out, qmin, qmax);
        }
    }
    return ovf ? IQO_EOVERFLOW : IQO_OK;
}

/* Max pooling.
 * "Quantization" blog, section 量化激活函数: max/clip/concat-like operators are
 * passive (same scale and zero point in and out), so the max is taken on codes.
 * READING: taps outside the image are skipped. */
int iqo_maxpool2d(const int32_t *x, int n, int h, int w, int c, int k, int s, int p, int32_t *y) {
    if (n < 0 || h <= 0 || w <= 0 || c <= 0 || k <= 0 || s <= 0 || p < 0 || 2 * p > k - 1)
        return IQO_EINVAL;
    int oh = (h + 2 * p - k) / s + 1;
    int ow = (w + 2 * p - k) / s + 1;
    if (oh <= 0 || ow <= 0) return IQO_EINVAL;
    int64_t rows = (int64_t)n * oh * ow;
#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < rows; ++row) {
        int ni = (int)(row / ((int64_t)oh * ow));
        int oy = (int)((row / ow) % oh);
        int ox = (int)(row % ow);
        for (int ci = 0; ci < c; ++ci) {
            int32_t best = INT32_MIN;
            for (int ky = 0; ky < k; ++ky)
                for (int kx = 0; kx < k; ++kx) {
                    int iy = oy * s - p + ky, ix = ox * s - p + kx;
                    if (iy < 0 || iy >= h || ix < 0 || ix >= w) continue;
                    int32_t v = x[(((int64_t)ni * h + iy) * w + ix) * c + ci];
                    if (v > best) best = v;
                }
            y[row * c + ci] = best;
        }
    }
    return IQO_OK;
}

/* Explicit im2col, used only to cross-check the direct convolution.
 * MegEngine 4-bit article, section conv 算子優化, Fig. 5: the input is rearranged
 * into an (IC*FH*FW) x (N*OH*OW) matrix; here stored transposed, one row per
 * output pixel, K ordered (kh, kw, ci) to match OHWI weights. */
int iqo_im2col(const int32_t *x, int n, int h, int w, int c_in, int32_t z_in, int kh, int kw,
               int sh, int sw, int ph, int pw, int32_t *cols) {
    if (n < 0 || h <= 0 || w <= 0 || c_in <= 0 || kh <= 0 || kw <= 0 || sh <= 0 || sw <= 0 ||
        ph < 0 || pw < 0 || h + 2 * ph < kh || w + 2 * pw < kw)
        return IQO_EINVAL;
    int oh = (h + 2 * ph - kh) / sh + 1;
    int ow = (w + 2 * pw - kw) / sw + 1;
    int64_t rows = (int64_t)n * oh * ow;
    int64_t kdim = (int64_t)kh * kw * c_in;
#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < rows; ++row) {
        int ni = (int)(row / ((int64_t)oh * ow));
        int oy = (int)((row / ow) % oh);
        int ox = (int)(row % ow);
        for (int ky = 0; ky < kh; ++ky)
            for (int kx = 0; kx < kw; ++kx)
                for (int ci = 0; ci < c_in; ++ci) {
                    int iy = oy * sh - ph + ky, ix = ox * sw - pw + kx;
                    int inside = iy >= 0 && iy < h && ix >= 0 && ix < w;
                    cols[row * kdim + ((int64_t)ky * kw + kx) * c_in + ci] =
                        inside ? x[(((int64_t)ni * h + iy) * w + ix) * c_in + ci] : z_in;
                }
    }
    return IQO_OK;
}
