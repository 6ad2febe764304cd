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

__global__ __launch_bounds__(256) void dequantize_kernel(const DequantParams p) {
    const int64_t chunk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t e0 = chunk * 16;
    if (e0 >= p.total) return;
    const int n = (int)((p.total - e0) < 16 ? (p.total - e0) : 16);
    const bool four = p.qtype == T_INT4 || p.qtype == T_UINT4;
    uint32_t w[4] = {0, 0, 0, 0};
    if (n == 16) {
        if (four) {
            uint2 v = *reinterpret_cast<const uint2*>(p.q + e0 / 2);
            w[0] = v.x; w[1] = v.y;
        } else {
            uint4 v = *reinterpret_cast<const uint4*>(p.q + e0);
            w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
        }
    } else {
        const int nb = four ? n / 2 : n;
        const uint8_t* src = p.q + (four ? e0 / 2 : e0);
        for (int j = 0; j < nb; ++j) w[j >> 2] |= (uint32_t)src[j] << (8 * (j & 3));
    }
    float out[16];
    if (p.per_channel) {
        ChanCursor cur(e0, p.ch, p.inner);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            float centred = (float)(code_at(w, j, p.qtype) - p.zp[cur.c]);
            out[j] = centred * p.scale[cur.c];
            cur.next(p.ch, p.inner);
        }
    } else {
        const float s = p.scale[0];
        const int32_t z = p.zp[0];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            float centred = (float)(code_at(w, j, p.qtype) - z);
            out[j] = centred * s;
        }
    }
    if (n == 16) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            *reinterpret_cast<float4*>(p.x + e0 + 4 * j) = make_float4(out[4 * j], out[4 * j + 1], out[4 * j + 2], out[4 * j + 3]);
    } else {
        for (int j = 0; j < n; ++j) p.x[e0 + j] = out[j];
    }
}

// Byte-wise max of packed bytes via 16-bit lanes: even and odd bytes separately.
__device__ __forceinline__ uint32_t max_u8x4(uint32_t a, uint32_t b) {
    uint32_t ae = a & 0x00FF00FFu, ao = (a >> 8) & 0x00FF00FFu;
    uint32_t be = b & 0x00FF00FFu, bo = (b >> 8) & 0x00FF00FFu;
    uint32_t me = (ae & 0xFFFFu) > (be & 0xFFFFu) ? (ae & 0xFFFFu) : (be & 0xFFFFu);
    me |= ((ae >> 16) > (be >> 16) ? (ae >> 16) : (be >> 16)) << 16;
    uint32_t mo = (ao & 0xFFFFu) > (bo & 0xFFFFu) ? (ao & 0xFFFFu) : (bo & 0xFFFFu);
    mo |= ((ao >> 16) > (bo >> 16) ? (ao >> 16) : (bo >> 16)) << 16;
    return me | (mo << 8);
}

__global__ __launch_bounds__(256) void maxpool_kernel(const PoolParams p) {
    // thread -> (output pixel, 16-channel group); signed codes are biased by 0x80
    // so that an unsigned byte max orders them correctly.
    const int cg = p.c / 16;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = (int64_t)p.n * p.oh * p.ow * cg;
    if (t >= total) return;
    const int g = (int)(t % cg);
    const int64_t pix = t / cg;
    const int ox = (int)(pix % p.ow);
    const int oy = (int)((pix / p.ow) % p.oh);
    const int64_t n = pix / ((int64_t)p.ow * p.oh);
    const uint32_t bias = p.is_signed ? 0x80808080u : 0u;
    uint32_t m[4] = {0, 0, 0, 0};
    for (int ky = 0; ky < p.k; ++ky) {
        const int iy = oy * p.s - p.p + ky;
        if (iy < 0 || iy >= p.h) continue;
        for (int kx = 0; kx < p.k; ++kx) {
            const int ix = ox * p.s - p.p + kx;
            if (ix < 0 || ix >= p.w) continue;
            uint4 v = *reinterpret_cast<const uint4*>(p.x + ((n * p.h + iy) * p.w + ix) * p.c + g * 16);
            m[0] = max_u8x4(m[0], v.x ^ bias);
            m[1] = max_u8x4(m[1], v.y ^ bias);
            m[2] = max_u8x4(m[2], v.z ^ bias);
            m[3] = max_u8x4(m[3], v.w ^ bias);
        }
    }
    *reinterpret_cast<uint4*>(p.y + pix * p.c + g * 16) = make_uint4(m[0] ^ bias, m[1] ^ bias, m[2] ^ bias, m[3] ^ bias);
}

// Quantize into a spatially padded NHWC tensor with c_pad >= c channels: every
// border pixel and every extra channel holds the zero-point code (the real value 0),
// which is what a convolution's zero padding means in the quantized domain.  One
// thread per output pixel.
__global__ __launch_bounds__(256) void quantize_pad_kernel(const QuantPadParams p) {
    const int hp = p.h + 2 * p.pad, wp = p.w + 2 * p.pad;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = (int64_t)p.n * hp * wp;
    if (t >= total) return;
    const int x = (int)(t % wp);
    const int y = (int)((t / wp) % hp);
    const int64_t n = t / ((int64_t)wp * hp);
    const int iy = y - p.pad, ix = x - p.pad;
    const bool inside = iy >= 0 && iy < p.h && ix >= 0 && ix < p.w;
    const float* src = p.x + ((n * p.h + iy) * p.w + ix) * p.c;
    uint8_t* dst = p.q + t * p.c_pad;
    for (int c = 0; c < p.c_pad; ++c) {
        const int32_t z = p.per_channel ? p.zp[c < p.c ? c : 0] : p.zp[0];
        int32_t q = z;
        if (inside && c < p.c) {
            const float s = p.per_channel ? p.scale[c] : p.scale[0];
            q = quant_one(src[c], s, z, p.qmin, p.qmax);
        }
        dst[c] = (uint8_t)(q & 0xFF);
    }
}

}  // namespace

hipError_t launch_quantize_pad(const QuantPadParams& p, hipStream_t stream) {
    const int64_t total = (int64_t)p.n * (p.h + 2 * p.pad) * (p.w + 2 * p.pad);
    if (total == 0) return hipSuccess;
    const int64_t blocks = (total + 255) / 256;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
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
    const int64_t chunks = (p.total + 15) / 16;
    if (chunks == 0) return hipSuccess;
    const int64_t blocks = (chunks + 255) / 256;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(dequantize_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_maxpool(const PoolParams& p, hipStream_t stream) {
    const int64_t total = (int64_t)p.n * p.oh * p.ow * (p.c / 16);
    if (total == 0) return hipSuccess;
    const int64_t blocks = (total + 255) / 256;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(maxpool_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace iqnn
