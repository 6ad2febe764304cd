// elementwise.hip -- quantize, dequantize and max pooling on gfx950.
//
// All three are HBM-bound streams: each thread owns 16 consecutive elements so
// every global access is a 16-byte (or 8-byte, for nibble-packed codes) vector
// access, and the arithmetic stays in registers.
//
// Quantize follows the "Quantization" blog, section 量化算子 (basic formula:
// round(value / scale), clip) and section 量化模式 (asymmetric: the offset is added
// after rounding); dequantize its section 反量化算子 and the MegEngine 4-bit
// article's r = S (Q - Z) (section 背景).  Division is IEEE correctly rounded
// (built with -fhip-fp32-correctly-rounded-divide-sqrt), rounding is half to even
// (v_rndne_f32).  Max pooling is passive ("Quantization" blog, 量化激活函数): the
// max is taken on codes, which keeps scale and zero point.
#include <hip/hip_runtime.h>
#include <algorithm>
#include <stdint.h>

#include "iqnn_internal.h"

#pragma clang fp contract(off)

namespace iqnn {
namespace {

// Channel cursor over the flattened [outer][ch][inner] view.
struct ChanCursor {
    int64_t c, i;
    __device__ ChanCursor(int64_t e, int64_t ch, int64_t inner) {
        int64_t t = e / inner;
        i = e - t * inner;
        c = t % ch;
    }
    __device__ void next(int64_t ch, int64_t inner) {
        if (++i == inner) {
            i = 0;
            if (++c == ch) c = 0;
        }
    }
};

__device__ __forceinline__ int32_t quant_one(float x, float s, int32_t z, int32_t qmin, int32_t qmax) {
    float r = __builtin_rintf(x / s);
    r = fminf(fmaxf(r, (float)(qmin - z)), (float)(qmax - z));
    return (int32_t)r + z;
}

__global__ __launch_bounds__(256) void quantize_kernel(const QuantParams p) {
    const int64_t chunk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t e0 = chunk * 16;
    if (e0 >= p.total) return;
    const int n = (int)((p.total - e0) < 16 ? (p.total - e0) : 16);
    float v[16];
    if (n == 16) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float4 f = *reinterpret_cast<const float4*>(p.x + e0 + 4 * j);
            v[4 * j] = f.x; v[4 * j + 1] = f.y; v[4 * j + 2] = f.z; v[4 * j + 3] = f.w;
        }
    } else {
        for (int j = 0; j < 16; ++j) v[j] = j < n ? p.x[e0 + j] : 0.0f;
    }
    int32_t q[16];
    if (p.per_channel) {
        ChanCursor cur(e0, p.ch, p.inner);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            q[j] = quant_one(v[j], p.scale[cur.c], p.zp[cur.c], p.qmin, p.qmax);
            cur.next(p.ch, p.inner);
        }
    } else {
        const float s = p.scale[0];
        const int32_t z = p.zp[0];
#pragma unroll
        for (int j = 0; j < 16; ++j) q[j] = quant_one(v[j], s, z, p.qmin, p.qmax);
    }
    if (p.qtype == T_INT8 || p.qtype == T_UINT8) {
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            w[j] = (uint32_t)(q[4 * j] & 0xFF) | ((uint32_t)(q[4 * j + 1] & 0xFF) << 8) |
                   ((uint32_t)(q[4 * j + 2] & 0xFF) << 16) | ((uint32_t)(q[4 * j + 3] & 0xFF) << 24);
        if (n == 16) {
            *reinterpret_cast<uint4*>(p.q + e0) = make_uint4(w[0], w[1], w[2], w[3]);
        } else {
            for (int j = 0; j < n; ++j) p.q[e0 + j] = (uint8_t)((w[j >> 2] >> (8 * (j & 3))) & 0xFF);
        }
    } else {
        uint32_t w[2] = {0, 0};
#pragma unroll
        for (int j = 0; j < 16; ++j) w[j >> 3] |= (uint32_t)(q[j] & 0xF) << (4 * (j & 7));
        if (n == 16) {
            *reinterpret_cast<uint2*>(p.q + e0 / 2) = make_uint2(w[0], w[1]);
        } else {
            for (int j = 0; j < n / 2; ++j) p.q[e0 / 2 + j] = (uint8_t)((w[j >> 2] >> (8 * (j & 3))) & 0xFF);
        }
    }
}

__device__ __forceinline__ int32_t code_at(const uint32_t* w, int j, int32_t qtype) {
    if (qtype == T_UINT8) return (int32_t)((w[j >> 2] >> (8 * (j & 3))) & 0xFF);
    if (qtype == T_INT8) return (int32_t)(int8_t)((w[j >> 2] >> (8 * (j & 3))) & 0xFF);
    int32_t nib = (int32_t)((w[j >> 3] >> (4 * (j & 7))) & 0xF);
    if (qtype == T_INT4 && nib >= 8) nib -= 16;
    return nib;
}

// One thread per 4 elements, so a wave's float4 stores are 1 KB contiguous; QT and
// PC (per-channel parameters) fixed per instantiation.
template <int QT, bool PC>
__global__ __launch_bounds__(256) void dequantize_kernel(const DequantParams p) {
    const int64_t e0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (e0 >= p.total) return;
    const int n = (int)((p.total - e0) < 4 ? (p.total - e0) : 4);
    constexpr bool four = QT == T_INT4 || QT == T_UINT4;
    uint32_t w[1] = {0};
    if (n == 4) {
        if (four) w[0] = *reinterpret_cast<const uint16_t*>(p.q + e0 / 2);
        else w[0] = *reinterpret_cast<const uint32_t*>(p.q + e0);
    } else {
        const int nb = four ? n / 2 : n;
        const uint8_t* src = p.q + (four ? e0 / 2 : e0);
        for (int j = 0; j < nb; ++j) w[0] |= (uint32_t)src[j] << (8 * j);
    }
    float out[4];
    if (PC) {
        ChanCursor cur(e0, p.ch, p.inner);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float centred = (float)(code_at(w, j, QT) - p.zp[cur.c]);
            out[j] = centred * p.scale[cur.c];
            cur.next(p.ch, p.inner);
        }
    } else {
        const float s = p.scale[0];
        const int32_t z = p.zp[0];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float centred = (float)(code_at(w, j, QT) - z);
            out[j] = centred * s;
        }
    }
    if (n == 4) {
        *reinterpret_cast<float4*>(p.x + e0) = make_float4(out[0], out[1], out[2], out[3]);
    } else {
        for (int j = 0; j < n; ++j) p.x[e0 + j] = out[j];
    }
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Max pooling over 16-channel groups: thread -> (output pixel, group).  The running
// maximum of each 32-bit word is kept as its even and odd bytes in two pairs of
// 16-bit lanes, so one packed 16-bit max (v_pk_max_u16) covers two bytes.  Signed
// codes are biased by 0x80 so that the unsigned order is the signed order.
// Indices are 32-bit (the host checks N*OH*OW*C/16 < 2^31).
__global__ __launch_bounds__(256) void maxpool_kernel(const PoolParams p) {
    const uint32_t cg = (uint32_t)p.c / 16;
    const uint32_t t = blockIdx.x * blockDim.x + threadIdx.x;
    const uint32_t total = (uint32_t)p.n * p.oh * p.ow * cg;
    if (t >= total) return;
    const uint32_t pix = t / cg, g = t - pix * cg;
    const uint32_t ohw = (uint32_t)p.oh * p.ow;
    const uint32_t n = pix / ohw, rem = pix - n * ohw;
    const uint32_t oy = rem / (uint32_t)p.ow, ox = rem - oy * (uint32_t)p.ow;
    const uint32_t bias = p.is_signed ? 0x80808080u : 0u;
    u16x2 me[4], mo[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) { me[d] = u16x2{0, 0}; mo[d] = u16x2{0, 0}; }
    const uint8_t* img = p.x + (int64_t)n * p.h * p.w * p.c + g * 16;
    for (int ky = 0; ky < p.k; ++ky) {
        const int iy = (int)oy * p.s - p.p + ky;
        if (iy < 0 || iy >= p.h) continue;
        for (int kx = 0; kx < p.k; ++kx) {
            const int ix = (int)ox * p.s - p.p + kx;
            if (ix < 0 || ix >= p.w) continue;
            const uint4 v = *reinterpret_cast<const uint4*>(img + ((int64_t)iy * p.w + ix) * p.c);
            const uint32_t vw[4] = {v.x ^ bias, v.y ^ bias, v.z ^ bias, v.w ^ bias};
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                me[d] = __builtin_elementwise_max(me[d], __builtin_bit_cast(u16x2, vw[d] & 0x00FF00FFu));
                mo[d] = __builtin_elementwise_max(mo[d], __builtin_bit_cast(u16x2, (vw[d] >> 8) & 0x00FF00FFu));
            }
        }
    }
    uint32_t r[4];
#pragma unroll
    for (int d = 0; d < 4; ++d)
        r[d] = (__builtin_bit_cast(uint32_t, me[d]) | (__builtin_bit_cast(uint32_t, mo[d]) << 8)) ^ bias;
    *reinterpret_cast<uint4*>(p.y + (int64_t)pix * p.c + g * 16) = make_uint4(r[0], r[1], r[2], r[3]);
}

// Quantize into a spatially padded NHWC tensor with c_pad >= c channels: every
// border pixel and every extra channel holds the zero-point code (the real value 0),
// which is what a convolution's zero padding means in the quantized domain.
// One thread per padded pixel; with c_pad == 4 the pixel is one 32-bit store.
// Indices are 32-bit (the host checks N*(H+2p)*(W+2p) < 2^31).
__global__ __launch_bounds__(256) void quantize_pad_kernel(const QuantPadParams p) {
    const uint32_t hp = (uint32_t)(p.h + 2 * p.pad), wp = (uint32_t)(p.w + 2 * p.pad);
    const uint32_t t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= (uint32_t)p.n * hp * wp) return;
    const uint32_t row = t / wp, x = t - row * wp;
    const uint32_t n = row / hp, y = row - n * hp;
    const int iy = (int)y - p.pad, ix = (int)x - p.pad;
    const bool inside = iy >= 0 && iy < p.h && ix >= 0 && ix < p.w;
    const float* src = p.x + (((int64_t)n * p.h + iy) * p.w + ix) * p.c;
    uint8_t* dst = p.q + (int64_t)t * p.c_pad;
    if (p.c_pad == 4) {
        uint32_t word = 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int32_t z = p.per_channel ? p.zp[c < p.c ? c : 0] : p.zp[0];
            int32_t q = z;
            if (inside && c < p.c) q = quant_one(src[c], p.per_channel ? p.scale[c] : p.scale[0], z, p.qmin, p.qmax);
            word |= (uint32_t)(q & 0xFF) << (8 * c);
        }
        *reinterpret_cast<uint32_t*>(dst) = word;
    } else {
        for (int c = 0; c < p.c_pad; ++c) {
            const int32_t z = p.per_channel ? p.zp[c < p.c ? c : 0] : p.zp[0];
            int32_t q = z;
            if (inside && c < p.c) q = quant_one(src[c], p.per_channel ? p.scale[c] : p.scale[0], z, p.qmin, p.qmax);
            dst[c] = (uint8_t)(q & 0xFF);
        }
    }
}

// The image case of quantize_pad_kernel: 3 channels padded to 4, one scale and zero
// point, W % 4 == 0 and a 16-byte aligned input.  A workgroup of 64 threads per
// run of a padded row: on an image row, thread g < W/4 quantizes source pixels
// 4g .. 4g+3 (48 contiguous bytes, three 16-byte loads) into four padded pixels and
// thread W/4 writes the row's left and right borders; on a border row every thread
// writes four pixels of zero-point codes.  The arithmetic per element is
// quantize_pad_kernel's.
__global__ __launch_bounds__(64) void quantize_pad3_kernel(const QuantPadParams p, int32_t blocks_per_row) {
    const int hp = p.h + 2 * p.pad, wp = p.w + 2 * p.pad;
    const int row = (int)blockIdx.x / blocks_per_row;           // n * hp + y
    const int g = ((int)blockIdx.x - row * blocks_per_row) * 64 + (int)threadIdx.x;
    const int n = row / hp, y = row - n * hp;
    const float s = p.scale[0];
    const int32_t z = p.zp[0];
    const uint32_t zb = (uint32_t)z & 0xFFu;
    const uint32_t zword = zb * 0x01010101u;
    uint32_t* drow = reinterpret_cast<uint32_t*>(p.q) + (int64_t)row * wp;   // one word per padded pixel
    const int iy = y - p.pad;
    if (iy < 0 || iy >= p.h) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (4 * g + k < wp) drow[4 * g + k] = zword;
        return;
    }
    const int groups = p.w / 4;
    if (g < groups) {
        const float4* src = reinterpret_cast<const float4*>(p.x + ((int64_t)(n * p.h + iy) * p.w + 4 * g) * 3);
        const float4 a = src[0], b = src[1], c = src[2];
        const float v[12] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w, c.x, c.y, c.z, c.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t q0 = (uint32_t)quant_one(v[3 * k], s, z, p.qmin, p.qmax) & 0xFFu;
            const uint32_t q1 = (uint32_t)quant_one(v[3 * k + 1], s, z, p.qmin, p.qmax) & 0xFFu;
            const uint32_t q2 = (uint32_t)quant_one(v[3 * k + 2], s, z, p.qmin, p.qmax) & 0xFFu;
            drow[p.pad + 4 * g + k] = q0 | (q1 << 8) | (q2 << 16) | (zb << 24);
        }
    } else if (g == groups) {
        for (int xo = 0; xo < p.pad; ++xo) {
            drow[xo] = zword;
            drow[p.pad + p.w + xo] = zword;
        }
    }
}

}  // namespace

hipError_t launch_quantize_pad(const QuantPadParams& p, hipStream_t stream) {
    const int64_t total = (int64_t)p.n * (p.h + 2 * p.pad) * (p.w + 2 * p.pad);
    if (total == 0) return hipSuccess;
    if (total >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    if (p.c == 3 && p.c_pad == 4 && !p.per_channel && p.w % 4 == 0 && (reinterpret_cast<uintptr_t>(p.x) & 15) == 0) {
        const int64_t wp = p.w + 2 * p.pad;
        const int64_t threads = std::max<int64_t>(p.w / 4 + 1, (wp + 3) / 4);   // per padded row
        const int64_t bpr = (threads + 63) / 64;
        const int64_t blocks = (int64_t)p.n * (p.h + 2 * p.pad) * bpr;
        if (blocks >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
        hipLaunchKernelGGL(quantize_pad3_kernel, dim3((unsigned)blocks), dim3(64), 0, stream, p, (int32_t)bpr);
        return hipGetLastError();
    }
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(quantize_pad_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_quantize(const QuantParams& p, hipStream_t stream) {
    const int64_t chunks = (p.total + 15) / 16;
    if (chunks == 0) return hipSuccess;
    const int64_t blocks = (chunks + 255) / 256;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_dequantize(const DequantParams& p, hipStream_t stream) {
    const int64_t chunks = (p.total + 3) / 4;
    if (chunks == 0) return hipSuccess;
    const int64_t blocks = (chunks + 255) / 256;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    const dim3 g((unsigned)blocks), b(256);
#define IQNN_DEQ(QT)                                                                          \
    if (p.qtype == QT) {                                                                      \
        if (p.per_channel) hipLaunchKernelGGL((dequantize_kernel<QT, true>), g, b, 0, stream, p); \
        else hipLaunchKernelGGL((dequantize_kernel<QT, false>), g, b, 0, stream, p);        \
        return hipGetLastError();                                                             \
    }
    IQNN_DEQ(T_INT8)
    IQNN_DEQ(T_UINT8)
    IQNN_DEQ(T_INT4)
    IQNN_DEQ(T_UINT4)
#undef IQNN_DEQ
    return hipErrorInvalidValue;
}

hipError_t launch_maxpool(const PoolParams& p, hipStream_t stream) {
    const int64_t total = (int64_t)p.n * p.oh * p.ow * (p.c / 16);
    if (total == 0) return hipSuccess;
    if (total >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(maxpool_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace iqnn
