// iqnn_internal.h -- parameter blocks and launchers shared by the host API and
// the gfx950 kernels of libiqnn.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace iqnn {

// Element types, same numbering as iqnn_dtype.
enum : int32_t { T_INT8 = 0, T_UINT8 = 1, T_INT4 = 2, T_UINT4 = 3, T_INT32 = 4 };
enum : int32_t { E_NONE = 0, E_RELU = 1, E_ADD = 2, E_ADD_RELU = 3, E_RAW = 4 };

// Activation gather modes of the implicit-GEMM kernel.
enum : int32_t {
    GATHER_B8 = 0,     // 8-bit codes, C_in % 16 == 0: one 16-byte load per K segment
    GATHER_B4 = 1,     // 4-bit codes, C_in % 16 == 0: one 8-byte load, unpacked to 16 int8
    GATHER_B8_ELEM = 2 // 8-bit codes, any C_in: element-wise gather (e.g. a 3-channel stem)
};

// Geometry of the prepacked layer buffer (device).  All offsets in bytes.
//   [0, 4*ocp)            int32  folded bias per output channel (physical order)
//   [4*ocp, 8*ocp)        float  requant multiplier M[c]
//   [8*ocp, 8*ocp+256)    float  M_res, padding
//   [w_off, w_off+ocp*kp) int8   weights, rows in kernel order, K padded to kp
struct PackGeom {
    int32_t ocp;    // output channels padded to a multiple of kOcPad
    int32_t kp;     // K padded to a multiple of kKPad
    int64_t w_off;
    int64_t bytes;
};

constexpr int kOcPad = 256;   // largest block extent along output channels
constexpr int kKPad = 64;     // one MFMA K step
constexpr int kBK = 128;      // K elements staged per pipeline step

PackGeom pack_geom(int64_t c_out, int64_t k);

// Position of physical output channel `oc` in the packed weight rows.  Each wave
// owns 64 channels as four 16-row MFMA tiles; lane group g of the 16x16 MFMA
// accumulator holds rows 4g..4g+3 of every tile.  Swapping the tile index and the
// lane-group index inside each 64-channel block makes the 16 values one lane holds
// 16 consecutive physical channels.
inline int32_t packed_row_of_channel(int32_t oc) {
    int32_t blk = oc & ~63, w = oc & 63;
    int32_t g = w >> 4, t = (w >> 2) & 3, r = w & 3;
    return blk + t * 16 + g * 4 + r;
}

struct ConvParams {
    const uint8_t* x;
    const int8_t* w;          // packed weights [ocp][kp]
    const int32_t* bias;      // [ocp]
    const float* mult;        // [ocp]
    const uint8_t* res;       // residual codes or nullptr
    uint8_t* y;
    int64_t m;                // output pixels N*OH*OW
    int32_t h, w_in, c;       // input H, W, C (elements)
    int32_t oh, ow;
    int32_t kh, kw, sh, sw, ph, pw;
    int32_t k;                // KH*KW*C
    int32_t kp;               // padded K = weight row stride (bytes)
    int32_t c_out;
    int32_t n_oc_tiles;
    uint32_t pad_word;        // four copies of the staged padding byte
    uint32_t x_xor;           // 0x80808080 for UINT8 activations, else 0
    int32_t x_signed4;        // INT4 activations: sign-extend nibbles
    int32_t y_type, res_type, epi;
    int32_t z_out, z_res;
    const float* m_res;       // residual multiplier S_res/S_out (in the packed buffer)
    float lo, hi;             // clip bounds minus z_out, as floats
    int32_t vec_store;        // C_out % 16 == 0: vector stores
};

hipError_t launch_qconv(const ConvParams& p, int gather, bool is_1x1, hipStream_t stream);

struct QuantParams {
    const float* x;
    uint8_t* q;
    const float* scale;
    const int32_t* zp;
    int64_t total, ch, inner;
    int32_t per_channel;
    int32_t qtype;
    int32_t qmin, qmax;
};
hipError_t launch_quantize(const QuantParams& p, hipStream_t stream);

struct DequantParams {
    const uint8_t* q;
    float* x;
    const float* scale;
    const int32_t* zp;
    int64_t total, ch, inner;
    int32_t per_channel;
    int32_t qtype;
};
hipError_t launch_dequantize(const DequantParams& p, hipStream_t stream);

struct PoolParams {
    const uint8_t* x;
    uint8_t* y;
    int32_t n, h, w, c, k, s, p, oh, ow;
    int32_t is_signed;
};
hipError_t launch_maxpool(const PoolParams& p, hipStream_t stream);

}  // namespace iqnn
