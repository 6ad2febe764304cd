/*
 * iqo.h -- plain, slow CPU oracle for integer-quantized convolution and GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  This library is the checker the GPU library is
 * compared against byte for byte.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load it; the product path never does.  It
 * shares no code, header, table or constant with the GPU library.
 *
 * Every code here is a logical integer held in an int32_t (one element per
 * int32, 4-bit codes unpacked); packing to bytes/nibbles is a separate step.
 * Floating point is IEEE-754 binary32 with round-to-nearest-even, one rounding
 * per operation (built with -ffp-contract=off: no fused multiply-add).
 *
 * Sources (cited by page title and section in each function):
 *   "Quantization" blog (loveleaves.github.io/p/quantization)
 *   MegEngine 4-bit quantization article (m.xsypw.cn/d/1897816.html)
 *   FQ-ViT article (aijishu.com/a/1060000000395099)
 *   Horizon QAT tool talk (chedongxi.com/p/309944.html)
 *   Horizon J5 Transformer deployment lecture (m.zdjbc1.cn ... news-363246)
 */
#ifndef IQO_H
#define IQO_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Quantized types. */
enum { IQO_INT8 = 0, IQO_UINT8 = 1, IQO_INT4 = 2, IQO_UINT4 = 3, IQO_INT32 = 4 };

/* Fused epilogues: requant only, Conv_Relu, Conv_Add, Conv_Add_Relu, raw int32. */
enum { IQO_EPI_NONE = 0, IQO_EPI_RELU = 1, IQO_EPI_ADD = 2, IQO_EPI_ADD_RELU = 3, IQO_EPI_RAW = 4 };

/* Return codes. */
enum { IQO_OK = 0, IQO_EINVAL = 1, IQO_EOVERFLOW = 2 };

int iqo_num_threads(void);
void iqo_set_num_threads(int n);

/* [Q_MIN, Q_MAX] of a code type. */
int iqo_qrange(int qtype, int32_t *qmin, int32_t *qmax);

/* Quantize x viewed as [outer][ch][inner]: q = clip(rne(x / S) + Z, Q_MIN, Q_MAX).
 * per_channel: scale[ch], zp[ch] (activations NHWC: inner = 1; OHWI weights per
 * output channel: outer = 1, inner = KH*KW*C_in); else scale[0], zp[0]. */
int iqo_quantize(const float *x, int32_t *q, int64_t outer, int64_t ch, int64_t inner,
                 const float *scale, const int32_t *zp, int per_channel, int qtype);

/* Dequantize: x = (q - Z) * S, same [outer][ch][inner] view. */
int iqo_dequantize(const int32_t *q, float *x, int64_t outer, int64_t ch, int64_t inner,
                   const float *scale, const int32_t *zp, int per_channel);

/* Byte packing.  8-bit types: one code per byte (two's complement for INT8).
 * 4-bit types: element 2j in bits 0-3, element 2j+1 in bits 4-7; n must be even. */
int iqo_pack(const int32_t *q, uint8_t *bytes, int64_t n, int qtype);
int iqo_unpack(const uint8_t *bytes, int32_t *q, int64_t n, int qtype);

/* Quantization parameters of the fused epilogue. */
float iqo_requant_multiplier(float s_in, float s_w, float s_out);
float iqo_residual_multiplier(float s_res, float s_out);
/* bias_q = rne(b / (S_in * S_w)); IQO_EOVERFLOW if it leaves int32. */
int iqo_quantize_bias(float b, float s_in, float s_w, int32_t *bias_q);

/* Direct convolution, NHWC activations [n][h][w][c_in], OHWI weights [c_out][kh][kw][c_in],
 * acc [n][oh][ow][c_out] = bias_q[oc] + sum (x - z_in)(w - z_w); positions outside the
 * image hold the real value 0.  bias_q may be NULL.  Fails with IQO_EOVERFLOW if any
 * accumulator leaves int32. */
int iqo_conv2d_acc(const int32_t *x, int n, int h, int w, int c_in, int32_t z_in,
                   const int32_t *wt, int c_out, int kh, int kw, int32_t z_w,
                   int sh, int sw, int ph, int pw, const int32_t *bias_q, int64_t *acc);

/* Naive GEMM: acc[m][n] = bias_q[n] + sum_k (a[m][k] - z_a)(b[n][k] - z_b). */
int iqo_gemm_acc(const int32_t *a, int64_t m, int64_t k, int32_t z_a, const int32_t *b,
                 int64_t n, int32_t z_b, const int32_t *bias_q, int64_t *acc);

/* Requantizing epilogue over acc [rows][ch]; mult[ch] per output channel.
 * res [rows][ch] codes (ADD / ADD_RELU only).  out_qtype IQO_INT32 only with IQO_EPI_RAW. */
int iqo_requant(const int64_t *acc, int64_t rows, int64_t ch, const float *mult, int epi,
                const int32_t *res, int32_t z_res, float m_res, int32_t z_out, int out_qtype,
                int32_t *out);

/* Max pooling over NHWC codes; taps outside the image are ignored. */
int iqo_maxpool2d(const int32_t *x, int n, int h, int w, int c, int k, int s, int p, int32_t *y);

/* Explicit im2col: cols [n*oh*ow][kh*kw*c_in], K ordered (kh, kw, ci); pads hold z_in. */
int iqo_im2col(const int32_t *x, int n, int h, int w, int c_in, int32_t z_in, int kh, int kw,
               int sh, int sw, int ph, int pw, int32_t *cols);

#ifdef __cplusplus
}
#endif
#endif
