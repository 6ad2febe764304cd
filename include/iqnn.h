/*
 * iqnn.h -- C ABI of libiqnn: integer-quantized convolution and GEMM on AMD
 * Instinct MI355X (gfx950).
 *
 * What the library computes (sources are cited by page title and section):
 *   - Linear quantization q = clip(round(x / S) + Z, Q_MIN, Q_MAX) and its inverse
 *     x = (q - Z) * S, per tensor or per channel, symmetric (Z = 0) or asymmetric
 *     ("Quantization" blog, sections 量化算子 / 反量化算子 / 量化模式 /
 *     tensor量化与通道量化; MegEngine 4-bit article, section 背景, Fig. 1 and 2).
 *   - Quantized convolution as an implicit GEMM with int32 accumulation, the
 *     zero-point terms that are known before inference folded into an int32 bias,
 *     and the fused Conv / Conv_Relu / Conv_Add_Relu epilogue (MegEngine 4-bit
 *     article, sections 緩解精度下降, 算子融合優化 and conv 算子優化;
 *     "Quantization" blog, sections 量化乘法, 量化加法, 量化激活函数, 量化矩阵乘).
 *   - Quantized GEMM, the same operator with a 1x1 kernel (Horizon J5 lecture:
 *     Linear is a 1x1 conv).
 *   - Max pooling on codes, a passive operator ("Quantization" blog, 量化激活函数).
 *
 * Conventions shared by every entry point
 *   Status     Every call returns an iqnn_status.  On error nothing is launched,
 *              no output byte is written, and iqnn_last_error() (thread-local)
 *              describes the failure.  Nothing aborts or prints.
 *   Memory     The caller owns all memory.  Pointers named *_dev are device
 *              pointers (hipMalloc / PyTorch CUDA tensors); *_host are host
 *              pointers.  No forward entry point allocates device memory.
 *   Streams    `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *              Forward / quantize / dequantize / maxpool calls are asynchronous on
 *              it; prepack is blocking (it returns after its copy completes).
 *   Layouts    Activations are NHWC with C innermost.  Conv weights are OHWI
 *              [C_out][KH][KW][C_in] codes.  GEMM: A [M][K] row-major, B [N][K]
 *              row-major (weight layout), C = A * B^T stored [M][N].  4-bit tensors
 *              pack two consecutive elements of the flattened tensor per byte:
 *              element 2j in bits 0-3, element 2j+1 in bits 4-7; INT4 is two's
 *              complement.  Weight codes carry a per-tensor zero point z_w / z_b
 *              (INT8 / INT4 with zero point 0 are symmetric).
 *   Rounding   Every round is round-half-to-even ("Quantization" blog, 量化算子).
 *              Floating point is IEEE binary32, one rounding per operation, no
 *              fused multiply-add, so results are bit-exact and reproducible.
 *   Threading  The library keeps no mutable global state: every choice a call
 *              makes depends only on its arguments, and calls on different
 *              streams or threads are independent.
 */
#ifndef IQNN_H
#define IQNN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define IQNN_ABI_VERSION 5

typedef enum {
    IQNN_OK = 0,
    IQNN_ERR_INVALID_ARG = 1,  /* a size, type, zero point, scale or pointer is invalid */
    IQNN_ERR_UNSUPPORTED = 2,  /* valid, but a combination the library does not implement */
    IQNN_ERR_ALIGNMENT = 3,    /* a pointer or row does not meet the documented alignment */
    IQNN_ERR_OVERFLOW = 4,     /* folded bias or accumulator bound would leave int32; a range too wide for binary32 */
    IQNN_ERR_HIP = 5           /* the HIP runtime reported an error */
} iqnn_status;

/* Element types.  Code ranges: INT8 [-128,127], UINT8 [0,255], INT4 [-8,7],
 * UINT4 [0,15] (MegEngine 4-bit article, Fig. 1 / Fig. 2). */
typedef enum {
    IQNN_INT8 = 0,
    IQNN_UINT8 = 1,
    IQNN_INT4 = 2,
    IQNN_UINT4 = 3,
    IQNN_INT32 = 4,  /* raw accumulator output only */
    /* Weights only: INT8 codes, symmetric (z_w = 0), in which every group of four
     * consecutive K positions (four consecutive input channels of one filter tap;
     * four consecutive K of a GEMM row) holds at most two nonzero codes: 2:4
     * structured sparsity (Horizon QAT talk, section 三: sparse plus quantized
     * weights).  The codes are given dense (OHWI / [N][K], zeros included); prepack
     * keeps two codes per group with their positions and fails with
     * IQNN_ERR_INVALID_ARG naming the channel and group when a group has more than
     * two nonzero codes.  The forward result is that of the same codes as INT8; the
     * kernel contracts only the kept half (the sparse int8 MFMA).  Needs 8-bit
     * activations, C_in % 64 == 0 (GEMM: K % 64 == 0), KH*KW <= 64, N*OH*OW < 2^31,
     * the binary32 epilogue, and for ADD / ADD_RELU an 8-bit residual with
     * C_out % 16 == 0; otherwise IQNN_ERR_UNSUPPORTED. */
    IQNN_INT8_2OF4 = 5
} iqnn_dtype;

/* Fused epilogues (MegEngine 4-bit article, section 算子融合優化: Conv_Relu and
 * Conv_Add_Relu; "Quantization" blog, 常见计算图优化: conv-add fusion).
 * With a = acc + folded bias (int32), M[c] = S_in*S_w[c]/S_out, M_res = S_res/S_out:
 *   t = float(a) * M[c]
 *   ADD, ADD_RELU:  t = t + float(r - Z_res) * M_res
 *   RELU, ADD_RELU: t = max(t, 0)
 *   y = clip(rne(t) + Z_out, Q_MIN, Q_MAX)
 * RAW_INT32 stores a itself (y_type must be IQNN_INT32). */
typedef enum {
    IQNN_EPI_NONE = 0,
    IQNN_EPI_RELU = 1,
    IQNN_EPI_ADD = 2,
    IQNN_EPI_ADD_RELU = 3,
    IQNN_EPI_RAW_INT32 = 4,
    /* Flag, OR'ed into NONE or RELU: integer-only requantization for targets without
     * floating point ("Quantization" blog, 量化模式: integer (power of two)
     * quantization; FQ-ViT article, LayerNorm code: get_MN).  Prepack writes each
     * M[c] as M_c * 2^-N_c with N_c = clamp(7 - floor(log2 M[c]), 0, 31) and
     * M_c = clamp(floor(M[c] * 2^N_c), 0, 255) (floor(log2) = the binary exponent)
     * and stores M_c * 2^-N_c (exact in binary32) in the multiplier slot; the kernel
     * computes y = clip(rne((acc + bias) * M_c / 2^N_c) + Z_out) (rne: half to even;
     * RELU clamps at Z_out), exactly: the product is below 2^40 and is formed, scaled
     * and rounded by one binary64 fused multiply-add, whose single rounding is that
     * rne.  Not with ADD, ADD_RELU or RAW_INT32, nor with iqnn_qconv_maxpool_fwd
     * (IQNN_ERR_UNSUPPORTED). */
    IQNN_EPI_INT_REQUANT = 16
} iqnn_epilogue;

/* Convolution descriptor.  Dilation 1, groups 1.  Output size
 * OH = (H + 2*pad_h - KH)/stride_h + 1, OW likewise.
 * x_type: INT8, UINT8, INT4 or UINT4.  w_type: INT8, UINT8, INT4 or UINT4 with
 * the per-tensor weight zero point z_w (INT8 / INT4 with z_w = 0 are symmetric),
 * or INT8_2OF4 (2:4-sparse symmetric INT8, see iqnn_dtype).
 * y_type: INT8, UINT8, INT4, UINT4, or INT32 with IQNN_EPI_RAW_INT32.
 * res_type: type of the residual for ADD / ADD_RELU (8- or 4-bit), else ignored.
 * z_in / z_out / z_res / z_w: zero points, within the code range of their type.
 * 4-bit activations need C_in % 16 == 0.  8-bit activations with C_in == 4 and no
 * padding (an input from iqnn_quantize_pad) take a 4-taps-per-load gather; other
 * C_in % 16 != 0 take a slower element gather.
 * Asymmetric weights (MegEngine 4-bit article, 緩解精度下降: a nonzero Z_W adds
 * the term Z_W * sum_k Q(I) of each output pixel, which depends on the input and
 * cannot be folded into the bias).  The kernels hold weights as w - s_w with
 * s_w = 128 for UINT8 and 0 otherwise; when z_w != s_w the per-pixel term is
 * accumulated next to the contraction, which the streaming path does for 8-bit
 * activations with C_in % 64 == 0, KH*KW <= 64 and N*OH*OW < 2^31.  Other layers
 * with z_w != s_w return IQNN_ERR_UNSUPPORTED (descriptor checks of every call). */
typedef struct {
    int32_t n, h, w, c_in, c_out;
    int32_t kh, kw, stride_h, stride_w, pad_h, pad_w;
    int32_t x_type, w_type, y_type, res_type;
    int32_t epilogue;
    int32_t z_in, z_out, z_res;
    int32_t z_w;
} iqnn_conv_desc;

/* GEMM descriptor: C[M][N] = epilogue(A[M][K] * B[N][K]^T).  a_type is the
 * activation type (8- or 4-bit, zero point z_a), b_type the weight type with zero
 * point z_b (as w_type / z_w of a convolution; the per-pixel term needs K % 64 ==
 * 0), c_type / res_type / epilogue / z_out / z_res as for convolution. */
typedef struct {
    int64_t m, n, k;
    int32_t a_type, b_type, c_type, res_type;
    int32_t epilogue;
    int32_t z_a, z_out, z_res;
    int32_t z_b;
} iqnn_gemm_desc;

/* ---------------------------------------------------------------- misc */

/* Returns IQNN_ABI_VERSION of the built library. */
int iqnn_abi_version(void);

/* Static string naming a status code. */
const char *iqnn_status_str(iqnn_status status);

/* Message for the last failed call on this thread ("" if none).  The pointer
 * stays valid until the next library call on the same thread. */
const char *iqnn_last_error(void);

/* Kernel configuration of one forward call (iqnn_qconv_fwd_cfg, iqnn_qgemm_fwd_cfg):
 * for tuning sweeps and for tests that run every block configuration.  Every choice
 * computes identical results; only speed differs.
 *   tile = -1: the automatic per-layer choice (what iqnn_qconv_fwd / iqnn_qgemm_fwd do).
 *     0..6   the ring kernel with blocks of (channels x pixels) 0: 64x256, 1: 128x128,
 *            2: 128x256, 3: 256x128, 4: 256x256, 5: 128x128 (3-stage ring), 6: 64x128;
 *     7..17  the persistent streaming kernel, four waves per workgroup: 7: 64x128
 *            (12-stage ring), 8: 64x128 (6), 9: 128x128 (8), 10: 128x128 (4), 11: 64x256
 *            (3), 12: 256x128 (6), 13: 128x256 (6), 14: 128x128 (3, three blocks per
 *            CU), 15: 128x256 (3), 16: 256x128 (3), 17: 256x256 (4);
 *     18     the direct 3x3 kernel (64-channel 8-bit activations, 3x3 / stride 1 /
 *            pad 1 on 56-pixel rows, no residual) at any batch, where the automatic
 *            choice takes it from 512 two-row tiles up;
 *     19     the FP6 path for 4-bit activations with symmetric INT4 weights and
 *            64*K < 2^24: weights and activations as BF6 (e3m2) codes on the f8f6f4
 *            MFMA with fp32 accumulation of integers, exact (the 4-bit inference
 *            article's case for 4-bit compute; CDNA4 has no 4-bit integer MFMA);
 *     20..23 the streaming kernel with eight waves per workgroup, one workgroup per
 *            CU: 20: 256x256 (4-stage ring), 21: 128x512 (3), 22: 256x128 (4),
 *            23: 512x128 (3).
 *   Layers a configuration cannot take (4-bit activations, C_in % 64 != 0, residual
 *   layouts it does not stream) keep a configuration that can.
 *   xcd_groups = 0: the automatic split of the streaming kernel's channel tiles across
 *     the eight XCDs; 1, 2, 4 or 8 force that many channel-tile groups.
 * Other values are IQNN_ERR_INVALID_ARG (before any launch). */
typedef struct {
    int32_t tile;
    int32_t xcd_groups;
} iqnn_kernel_cfg;

/* ------------------------------------------------------- quantize / dequantize */

/* Quantization parameters of a tensor from its real range [minv, maxv] (host, pure
 * function).  MinMax uniform quantization (FQ-ViT article, §3.1); the Horizon QAT
 * talk (section 三) fixes a scale from the real min / max over the INT8 range.
 * Every step is one binary32 operation rounded to nearest even:
 *   symmetric (signed qtype only): S = max(|minv|, |maxv|) / Q_MAX, Z = 0;
 *   asymmetric: the range is widened to hold 0 (mn = min(minv, 0), mx = max(maxv, 0)),
 *   S = (mx - mn) / (Q_MAX - Q_MIN), Z = clip(Q_MIN - rne(mn / S), Q_MIN, Q_MAX),
 *   so the real 0 has the exact code Z.
 * A scale below the smallest normal binary32 (a zero range) is replaced by 1, so every
 * value of such a tensor quantizes to Z.  qtype: INT8, UINT8, INT4, UINT4.  Errors:
 * IQNN_ERR_INVALID_ARG for null outputs, non-finite bounds, minv > maxv, another
 * qtype, or symmetric with an unsigned qtype; IQNN_ERR_OVERFLOW when mx - mn is not a
 * finite binary32.  Outputs are written only on success. */
iqnn_status iqnn_choose_qparams(float minv, float maxv, int32_t qtype, int symmetric, float *scale,
                                int32_t *zp);


/* Quantize fp32 -> codes.  x viewed as [outer][ch][inner]; with per_channel the
 * scale and zero point of element (o, c, i) are scale_dev[c], zp_dev[c], else
 * scale_dev[0], zp_dev[0].  q = clip(rne(x / S) + Z, Q_MIN, Q_MAX) with one IEEE
 * division ("Quantization" blog, 量化算子 and 量化模式).  qtype: INT8, UINT8, INT4,
 * UINT4; 4-bit output packs element pairs of the flattened tensor, so
 * outer*ch*inner must be even.  Infinities saturate; NaN inputs give unspecified
 * codes.  Scales and zero points are read on the device at run time; they must
 * be positive finite floats and zero points within the code range.
 * Alignment: x_dev 16 bytes, q_dev 16 bytes (8-bit) or 8 bytes (4-bit). */
iqnn_status iqnn_quantize(const float *x_dev, void *q_dev, int64_t outer, int64_t ch,
                          int64_t inner, const float *scale_dev, const int32_t *zp_dev,
                          int per_channel, int32_t qtype, void *stream);

/* Dequantize codes -> fp32: x = float(q - Z) * S ("Quantization" blog, 反量化算子;
 * MegEngine 4-bit article, 背景).  Same views, types and alignment as quantize. */
iqnn_status iqnn_dequantize(const void *q_dev, float *x_dev, int64_t outer, int64_t ch,
                            int64_t inner, const float *scale_dev, const int32_t *zp_dev,
                            int per_channel, int32_t qtype, void *stream);

/* Quantize an fp32 NHWC tensor [n][h][w][c] into codes laid out
 * [n][h+2*pad][w+2*pad][c_pad] (c_pad >= c): interior elements are quantized as by
 * iqnn_quantize (per_channel: scale_dev[c], zp_dev[c] along the channel axis), and
 * every border pixel and every extra channel holds the zero-point code, i.e. the
 * real value 0.  A convolution with padding p over the unpadded tensor equals the
 * same convolution with padding 0 over this one (zero padding means real 0; an
 * extra channel multiplies a zero-valued input).  Used for image inputs: 3 channels
 * padded to 4 let the convolution load 4 taps x 4 channels per 16 bytes.
 * qtype: INT8 or UINT8.  Alignment: x_dev, q_dev 4 bytes.  Size: n*(h+2pad)*(w+2pad)
 * below 2^31 (IQNN_ERR_UNSUPPORTED otherwise). */
iqnn_status iqnn_quantize_pad(const float *x_dev, void *q_dev, int32_t n, int32_t h, int32_t w,
                              int32_t c, int32_t pad, int32_t c_pad, const float *scale_dev,
                              const int32_t *zp_dev, int per_channel, int32_t qtype, void *stream);

/* ---------------------------------------------------------------- convolution */

/* Bytes of device memory the prepacked form of this layer needs. 0 if the
 * descriptor is invalid (iqnn_last_error says why). */
size_t iqnn_qconv_packed_size(const iqnn_conv_desc *desc);

/* Prepack one conv layer (blocking; not for the hot path).
 * w_host: OHWI weight codes, one byte per code (INT8) or packed nibbles (INT4,
 *   C_in even).  bias_host: fp32 [C_out] or NULL.  s_in: input scale.  s_w_host:
 *   weight scales, [C_out] when per_channel else [1].  s_out: output scale.
 *   s_res: residual scale (ADD / ADD_RELU; ignored otherwise).
 * Computes, once: bias_q[c] = rne(B[c] / (S_in*S_w[c])) (MegEngine 4-bit article,
 *   緩解精度下降: terms known before inference go into the bias), the folded int32
 *   bias (bias_q[c] plus the Z_in and Z_in*Z_W terms, in the kernel's shifted
 *   operands; see iqnn_qconv_prepack_host), M[c] = (S_in*S_w[c])/S_out and M_res = S_res/S_out in binary32
 *   ("Quantization" blog, 量化乘法: the combined scale is precomputed), and the
 *   weights reordered for the kernel (output channels permuted so each lane stores
 *   contiguous channels: MegEngine 4-bit article, conv 算子優化, Fig. 8).
 * packed_dev: device buffer of iqnn_qconv_packed_size() bytes, 256-byte aligned.
 * Errors: INVALID_ARG (bad desc, code out of range, non-positive/non-finite scale,
 *   a multiplier M[c] or M_res that is not a normal float in [FLT_MIN, 1e20] -- the
 *   bound keeps every epilogue intermediate finite), OVERFLOW (folded bias or
 *   accumulator bound outside int32). */
iqnn_status iqnn_qconv_prepack(const iqnn_conv_desc *desc, const void *w_host,
                               const float *bias_host, float s_in, const float *s_w_host,
                               int per_channel, float s_out, float s_res, void *packed_dev,
                               size_t packed_bytes, void *stream);

/* Host-side prepack: writes into packed_host (iqnn_qconv_packed_size bytes) exactly
 * the bytes iqnn_qconv_prepack copies to the device, and makes no HIP call.  For
 * callers that prepack without a device, cache packed layers, or upload them on
 * their own stream.  Same arguments and errors as iqnn_qconv_prepack.
 * The packed form, with OCP = C_out rounded up to 256 and KP = K rounded up to 64
 * (K = KH*KW*C_in), is:
 *   int32 bias[OCP]     folded bias per physical output channel
 *   float mult[OCP]     requant multiplier M[c] (1.0 for RAW_INT32; M_c * 2^-N_c
 *                       for IQNN_EPI_INT_REQUANT)
 *   256-byte header:    float m_res at +0; 64 bytes holding the input zero-point
 *                       code (the row the kernel reads for padding) at +64; zeros
 *   int8  w[OCP][KP]    weight codes; row packed_row(c) holds channel c, where for
 *                       c = 32b + 16h + 4j + r, packed_row(c) = 32b + 8j + 4h + r;
 *                       for 4-bit activations the K positions inside every group of
 *                       16 are ordered 0,2,4,6,1,3,5,7,8,10,12,14,9,11,13,15
 *                       (the order the kernel unpacks nibbles in); zero padding;
 *   then, for layers the streaming kernel runs, regions whose layout is internal to
 *   the library (a tile-order copy of the weights -- INT4 weights of 4-bit layers
 *   kept two to a byte there --, the 2:4 blocks, the BF6 copy of the FP6 path);
 *   iqnn_qconv_packed_size counts them.
 * The kernel contracts a = q_I - s (s = 128 for UINT8 activations, else 0) with the
 * stored weights b = q_W - s_w (s_w = 128 for UINT8 weights, else 0), so
 *   sum_k (q_I - Z_in)(q_W - Z_w) = sum a*b + (s - Z_in) sum_k b + K (s - Z_in)(s_w - Z_w)
 *                                   + (s_w - Z_w) sum_k a,
 * and the folded bias is rne(B[c]/(S_in*S_w[c])) + (s - Z_in)*sum_k b[c][k]
 * + K*(s - Z_in)*(s_w - Z_w); the last term, per output pixel, is the kernel's. */
iqnn_status iqnn_qconv_prepack_host(const iqnn_conv_desc *desc, const void *w_host,
                                    const float *bias_host, float s_in, const float *s_w_host,
                                    int per_channel, float s_out, float s_res, void *packed_host,
                                    size_t packed_bytes);

/* Quantized conv forward: y = epilogue(conv(x, W) + folded bias).
 * x_dev: NHWC codes of x_type.  packed_dev: from iqnn_qconv_prepack with the same
 * descriptor.  res_dev: NHWC [N][OH][OW][C_out] codes of res_type for ADD /
 * ADD_RELU, NULL otherwise.  y_dev: NHWC [N][OH][OW][C_out] of y_type.
 * Padding positions hold the real value 0 (code Z_in).  Implicit GEMM: no im2col
 * buffer, no workspace.  Alignment: x, y, res 16 bytes. */
iqnn_status iqnn_qconv_fwd(const iqnn_conv_desc *desc, const void *x_dev,
                           const void *packed_dev, const void *res_dev, void *y_dev,
                           void *stream);

/* iqnn_qconv_fwd with an explicit kernel configuration (see iqnn_kernel_cfg); cfg NULL
 * is the automatic choice.  Same results, arguments and errors. */
iqnn_status iqnn_qconv_fwd_cfg(const iqnn_conv_desc *desc, const void *x_dev,
                               const void *packed_dev, const void *res_dev, void *y_dev,
                               const iqnn_kernel_cfg *cfg, void *stream);

/* Quantized conv followed by max pooling of its output codes, fused: the conv's
 * output is never written, only y_dev = maxpool(conv(x)) [N][PH][PW][C_out] with
 * PH = (OH + 2*pool_pad - pool_k)/pool_stride + 1, PW likewise.  Max pooling is
 * passive on codes ("Quantization" blog, 量化激活函数; the stem -> pooling step of
 * the ResNet-50 graph in the MegEngine 4-bit article, 算子融合優化, Fig. 3), so the
 * bytes equal iqnn_qconv_fwd followed by iqnn_maxpool2d.  Supported: the image stem
 * shape class -- 8-bit activations with C_in == 4 and no padding (an input from
 * iqnn_quantize_pad), stride 2, KH <= 8, KW <= 8, C_out == 64 with 8-bit codes,
 * Conv or Conv_Relu, symmetric weights (or z_w equal to the weight shift), an even
 * input width W, OH and OW even, OW <= 248, (KH+2)*W*4 <= 9200 (two output rows' input
 * rows fit one 9 KB LDS buffer), N*H*W*4 input bytes divisible by 16 (the kernel moves
 * whole 16-byte units), pool 3x3 stride 2 padding 1; IQNN_ERR_UNSUPPORTED
 * otherwise (validated before any launch).  Alignment: x, y 16 bytes; packed 256. */
iqnn_status iqnn_qconv_maxpool_fwd(const iqnn_conv_desc *desc, const void *x_dev,
                                   const void *packed_dev, void *y_dev, int32_t pool_k,
                                   int32_t pool_stride, int32_t pool_pad, void *stream);

/* Two quantized 1x1 convs where the second reads the first's output: y_a =
 * conv_a(x) (with res_dev for ADD / ADD_RELU) and y_b = conv_b(y_a), bytes equal to
 * iqnn_qconv_fwd(desc_a) followed by iqnn_qconv_fwd(desc_b) on y_a.  This is the
 * hand-off between two bottleneck blocks of the ResNet-50 graph (MegEngine 4-bit
 * article, 算子融合優化, Fig. 3 and 4: the Conv_Add_Relu that ends a block feeds the
 * next block's first Conv_Relu and its residual add).  desc_b's input must be
 * desc_a's output: N, H = OH_a, W = OW_a, C_in = C_out_a, x_type = y_type_a, z_in =
 * z_out_a (IQNN_ERR_INVALID_ARG otherwise).  Both outputs are written; y_a is also the
 * next block's residual.  One launch keeps y_a's codes in LDS for conv_b instead of
 * reading them back from HBM when: both convs are 1x1, stride 1, unpadded; conv_a 64
 * -> 256 channels with an 8-bit residual (ADD / ADD_RELU); conv_b 256 -> 64 or 128
 * channels (NONE / RELU); 8-bit activations and outputs, INT8 weights, binary32
 * requantization.  Every other valid pair runs as the two calls, with their errors.
 * Pointers and alignment as iqnn_qconv_fwd (packed_a_dev, packed_b_dev from
 * iqnn_qconv_prepack with desc_a, desc_b). */
iqnn_status iqnn_qconv_pair_fwd(const iqnn_conv_desc *desc_a, const iqnn_conv_desc *desc_b,
                                const void *x_dev, const void *packed_a_dev, const void *res_dev,
                                const void *packed_b_dev, void *y_a_dev, void *y_b_dev,
                                void *stream);

/* ---------------------------------------------------------------------- GEMM */

size_t iqnn_qgemm_packed_size(const iqnn_gemm_desc *desc);

/* As iqnn_qconv_prepack, for B [N][K] codes (INT8 bytes or INT4 nibbles, K even),
 * s_b_host [N] (per_channel) or [1]. */
iqnn_status iqnn_qgemm_prepack(const iqnn_gemm_desc *desc, const void *b_host,
                               const float *bias_host, float s_a, const float *s_b_host,
                               int per_channel, float s_out, float s_res, void *packed_dev,
                               size_t packed_bytes, void *stream);

/* Host-side GEMM prepack; see iqnn_qconv_prepack_host (B rows play the role of
 * output channels, K of KH*KW*C_in). */
iqnn_status iqnn_qgemm_prepack_host(const iqnn_gemm_desc *desc, const void *b_host,
                                    const float *bias_host, float s_a, const float *s_b_host,
                                    int per_channel, float s_out, float s_res, void *packed_host,
                                    size_t packed_bytes);

/* C[M][N] = epilogue(A[M][K] * B^T + folded bias) ("Quantization" blog, 量化矩阵乘:
 * int8 in, int32 accumulate, requantize to int8 out).  res_dev [M][N] or NULL. */
iqnn_status iqnn_qgemm_fwd(const iqnn_gemm_desc *desc, const void *a_dev,
                           const void *packed_dev, const void *res_dev, void *c_dev,
                           void *stream);

/* iqnn_qgemm_fwd with an explicit kernel configuration (see iqnn_kernel_cfg). */
iqnn_status iqnn_qgemm_fwd_cfg(const iqnn_gemm_desc *desc, const void *a_dev,
                               const void *packed_dev, const void *res_dev, void *c_dev,
                               const iqnn_kernel_cfg *cfg, void *stream);

/* -------------------------------------------------------------------- pooling */

/* Max pooling k x k, stride s, padding p over NHWC codes of dtype INT8 or UINT8;
 * taps outside the image are skipped (requires 2p <= k-1).  Passive: the output
 * keeps the input's scale and zero point ("Quantization" blog, 量化激活函数).
 * Alignment: x, y 16 bytes; C % 16 == 0; N*OH*OW*C/16 below 2^31
 * (IQNN_ERR_UNSUPPORTED otherwise). */
iqnn_status iqnn_maxpool2d(const void *x_dev, void *y_dev, int32_t n, int32_t h, int32_t w,
                           int32_t c, int32_t k, int32_t stride, int32_t pad, int32_t dtype,
                           void *stream);

/* ------------------------------------------------------- measurement helpers */

/* Calibration launches for reporting the kernels above against what this GPU
 * reaches, not part of the operator.  iqnn_probe_empty launches an empty kernel
 * (launch overhead).  iqnn_probe_mfma_rate launches `blocks` workgroups of four
 * waves, each wave running `iters` rounds of eight independent int8 32x32x32 MFMAs
 * from registers (2 * 32 * 32 * 32 * 8 * iters * 4 * blocks operations), and writes
 * blocks * 256 int32 sums to sink_dev (caller-owned device memory, 4-byte aligned).
 * Both are asynchronous on `stream`.  Errors: INVALID_ARG (non-positive iters /
 * blocks, null sink), ALIGNMENT, HIP. */
iqnn_status iqnn_probe_empty(void *stream);
iqnn_status iqnn_probe_mfma_rate(int32_t iters, int32_t blocks, int32_t *sink_dev, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* IQNN_H */
