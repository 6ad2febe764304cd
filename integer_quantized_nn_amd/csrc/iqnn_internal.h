// iqnn_internal.h -- parameter blocks and launchers shared by the host API and
// the gfx950 kernels of libiqnn.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace iqnn {

// Element types, same numbering as iqnn_dtype.
enum : int32_t { T_INT8 = 0, T_UINT8 = 1, T_INT4 = 2, T_UINT4 = 3, T_INT32 = 4, T_INT8_2OF4 = 5 };
enum : int32_t { E_NONE = 0, E_RELU = 1, E_ADD = 2, E_ADD_RELU = 3, E_RAW = 4 };

// Activation gather modes of the implicit-GEMM kernel.
enum : int32_t {
    GATHER_B8 = 0,     // 8-bit codes, C_in % 16 == 0: one 16-byte load per K segment
    GATHER_B4 = 1,     // 4-bit codes, C_in % 16 == 0: one 8-byte load, unpacked to 16 int8
    GATHER_B8_ELEM = 2, // 8-bit codes, any C_in: element-wise gather
    GATHER_C4 = 3,      // 8-bit codes, C_in == 4, no padding: one 16-byte load = 4 taps x 4 channels
    GATHER_B4S = 4      // 4-bit codes, C_in % 64 == 0: packed rows streamed to LDS, unpacked per fragment
};

// Geometry of the prepacked layer buffer (device).  All offsets in bytes.
//   [0, 4*ocp)            int32  folded bias per output channel (physical order)
//   [4*ocp, 8*ocp)        float  requant multiplier M[c]
//   [8*ocp, 8*ocp+256)    header: float M_res at +0, 64 pad-code bytes at +64
//   [w_off, w_off+ocp*kp) int8   weights, rows in kernel order, K padded to kp
//   2:4 weights (T_INT8_2OF4) use the first 5/8 of that region instead, as blocks of
//   kSpBlock bytes, one per (kSpRows-row channel tile, 64-K stage), tile-major: the
//   sparse kernel's LDS image of the stage (kept codes, then positions)
//   [t_off, t_off+ocp*kp) int8   the same weights in tile order for the streaming
//                                kernel: 4 KB blocks, one per (64-row group, 64-K
//                                stage), group-major; a block is the stage's LDS image
//                                (row r's 16-byte K segment q at slot q ^ ((r >> 2) & 3))
struct PackGeom {
    int32_t ocp;    // output channels padded to a multiple of kOcPad
    int32_t kp;     // K padded to a multiple of kKPad
    int64_t w_off;
    int64_t t_off;
    int64_t bytes;
};

constexpr int kOcPad = 256;   // largest block extent along output channels
constexpr int kKPad = 64;     // one MFMA K step
constexpr int kBK = 128;      // K elements staged per pipeline step
constexpr int kSpRows = 128;                  // 2:4 weights: channel rows per block
constexpr int kSpBlock = kSpRows * (32 + 8);  // 2:4 weights: bytes per (tile, stage) block

PackGeom pack_geom(int64_t c_out, int64_t k);

// Position of physical output channel `oc` in the packed weight rows.  A 32x32
// MFMA accumulator gives lane half h the rows 8j + 4h + r (j, r = 0..3) of its
// 32-row tile.  Storing channel 32b + 16h + 4j + r at row 32b + 8j + 4h + r makes
// the 16 values a lane holds 16 consecutive physical channels.
inline int32_t packed_row_of_channel(int32_t oc) {
    int32_t blk = oc & ~31, w = oc & 31;
    int32_t h = w >> 4, j = (w >> 2) & 3, r = w & 3;
    return blk + j * 8 + h * 4 + r;
}

// Byte offsets inside the packed layer header (after the two per-channel arrays).
constexpr int kHdrMres = 0;     // float M_res
constexpr int kHdrPad = 64;     // 64 bytes of the input zero-point code (the padding row)

struct ConvParams {
    const uint8_t* x;
    const int8_t* w;          // packed weights [ocp][kp]
    const int8_t* w_tiled;    // the same weights in 64-row, 64-K blocks (streaming kernel)
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
    int32_t n_px_tiles;       // set by the launcher
    int32_t group_px;         // pixel tiles per rasterization group (set by the launcher)
    int32_t gx;               // streaming kernel: workgroups per XCD (set by the launcher)
    int32_t px_chunk;         // streaming kernel: pixel tiles per XCD share (set by the launcher)
    int32_t xo_groups;        // streaming kernel: channel-tile groups across the XCDs (set by the launcher)
    int32_t xcd_force;        // 1, 2, 4 or 8: channel-tile groups asked for by the caller; 0: automatic
    uint32_t pad_word;        // four copies of the staged padding byte
    uint32_t x_xor;           // 0x80808080 for UINT8 activations, else 0
    int32_t x_signed4;        // INT4 activations: sign-extend nibbles
    int32_t y_type, res_type, epi;
    int32_t z_out, z_res;
    int32_t zw_red;           // s_w - Z_w: coefficient of the per-pixel activation sum (0: none)
    const float* m_res;       // residual multiplier S_res/S_out (in the packed buffer)
    const uint8_t* pad_row;   // 64 bytes of the raw input zero-point code (in the packed buffer)
    const uint8_t* w_idx;     // 2:4 weights: the positions of block 0 (non-null marks the 2:4 layout)
    // Epilogue constants (host-computed).  The requantized value is clipped to
    // [t_lo, t_hi] = [Q_MIN (or max(Q_MIN, Z_out) with ReLU), Q_MAX] - Z_out, then
    // out_magic = 1.5 * 2^23 + (Z_out minus its odd part) is added, which rounds to
    // nearest even; out_fix (the odd part of Z_out, 0 or 1) is added to the float's
    // bits, leaving the output code in the low byte.  Residual codes are read as
    // unsigned codes shifted by 128 (INT8) / 8 (INT4) / 0: (code ^ res_xor) - res_zf
    // == r - Z_res.
    // For 8-bit outputs whose code range excludes 0 (ReLU with Z_out >= 1, say) the
    // bytes before the fix never hold 0xFF, so the fix is added once per packed word:
    // out_fix4 = 0x01010101 and out_fix = 0.
    float t_lo, t_hi, out_magic;
    uint32_t out_fix, out_fix4;
    // Integer-only requantization: mult[c] holds M_c * 2^-N_c exactly (see
    // int_multiplier); the rounded value is clipped to [q_lo, q_hi] = [t_lo, t_hi] as
    // integers.
    int32_t int_rq, q_lo, q_hi;
    float res_zf;
    uint32_t res_xor;
    int32_t vec_store;        // C_out % 16 == 0: vector stores
    int32_t w4;               // 4-bit streaming layer whose tile-order copy holds packed INT4 weights
    int32_t f6;               // 4-bit streaming layer on the FP6 MFMA: bias and w_tiled point at the
                              // layer's BF6 region (set by the host, forced with kTileFp6)
};

// tile < 0 picks the kernel and its tile configuration from the layer shape; 0..17
// and 20..23 force a block configuration of the ring / streaming kernels,
// kTileDirect3x3 the direct 3x3 kernel on the layers it takes (2:4-sparse layers always
// take their own 128x128 configuration).  The caller's iqnn_kernel_cfg, per call.
constexpr int kTileDirect3x3 = 18;
constexpr int kTileFp6 = 19;   // 4-bit layers with INT4 weights: the FP6 MFMA path
constexpr int kMaxTile = 23;
hipError_t launch_qconv(const ConvParams& p, int gather, bool is_1x1, hipStream_t stream, int tile);

// The image stem (4-channel padding-free input, stride 2) fused with 3x3 / stride 2 /
// pad 1 max pooling of its codes into yp [N][OH/2][OW/2][64].
bool stem_pool_ok(const ConvParams& p);
hipError_t launch_stem_pool(const ConvParams& p, uint8_t* yp, hipStream_t stream);

// Two 1x1 convs over the same pixels, the second reading the first's output
// (y_b = conv_b(y_a)), in one launch: a.y is written and b.x is ignored.
bool pair_ok(const ConvParams& a, const ConvParams& b);
hipError_t launch_pair(const ConvParams& a, const ConvParams& b, hipStream_t stream);

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

struct QuantPadParams {
    const float* x;           // [n][h][w][c]
    uint8_t* q;               // [n][h+2*pad][w+2*pad][c_pad]
    const float* scale;
    const int32_t* zp;
    int32_t n, h, w, c, pad, c_pad;
    int32_t per_channel;
    int32_t qmin, qmax;
};
hipError_t launch_quantize_pad(const QuantPadParams& p, hipStream_t stream);

// Calibration kernels (probe.hip): an empty launch, and `blocks` workgroups of four
// waves running `iters` rounds of eight independent int8 MFMAs each (sink: blocks*256
// int32 results).
hipError_t launch_probe_empty(hipStream_t stream);
hipError_t launch_probe_mfma_rate(int32_t iters, int32_t blocks, int32_t* sink, hipStream_t stream);

struct PoolParams {
    const uint8_t* x;
    uint8_t* y;
    int32_t n, h, w, c, k, s, p, oh, ow;
    int32_t is_signed;
};
hipError_t launch_maxpool(const PoolParams& p, hipStream_t stream);

}  // namespace iqnn
