// qconv.hip -- implicit-GEMM quantized convolution / GEMM for gfx950 (CDNA4).
//
// The operator (MegEngine 4-bit article, sections 緩解精度下降, 算子融合優化 and
// conv 算子優化; "Quantization" blog, section 量化矩阵乘):
//   acc[p][oc] = sum_k A[p][k] * W[oc][k]            int8 x int8 -> int32 (MFMA)
//   a          = acc + bias_fold[oc]                  zero-point terms folded in
//   y[p][oc]   = epilogue(a)                          requant / ReLU / residual add
// where p runs over output pixels (n, oh, ow) and k over (kh, kw, ci).  The im2col
// matrix A is never built: each workgroup gathers its tile straight from the NHWC
// activations on the way into LDS, as the MegEngine article describes for its
// global->shared load (conv 算子優化, after Fig. 5).
//
// gfx950 design shared by the kernels below
//   * Contraction on v_mfma_i32_32x32x32_i8 (signed int8 only; 32 cycles per
//     instruction, so 5.0 POP/s at 2.4 GHz on 256 CUs -- a register-only loop
//     reaches 60-95 % of that, depending on the clock a GPU holds under MFMA
//     load, and iqnn_probe_mfma_rate measures it).  UINT8 activations
//     enter the MFMA as q - 128 (XOR 0x80); the host folds +128*sum(W) into the
//     bias.  4-bit activations are unpacked to int8 on chip (UINT4 zero-extended,
//     INT4 sign-extended): CDNA4 has no 4-bit integer MFMA, so 4-bit data saves HBM
//     bytes, not MFMA cycles.
//   * Output channels are the MFMA rows (A operand = weights), pixels the columns
//     (B operand = activations): the accumulator a lane holds runs along channels,
//     the NHWC-friendly orientation the MegEngine article gets by transposing its
//     output (conv 算子優化, Fig. 7 and after).  A 32x32 accumulator gives lane half
//     h the rows 8j+4h+r; the prepacked weight rows are permuted inside every
//     32-channel block (the column-permutation identity of the article's Fig. 8) so
//     those 16 values are 16 consecutive channels: one 16-byte store per pixel.
//   * 4 or 8 waves per workgroup.  Workgroup ids are remapped so consecutive tiles
//     land on the same XCD (ids are dealt round-robin over 8 XCDs, each with its own
//     L2).
//   * The epilogue runs in registers in strict binary32 (no contraction) with
//     round-half-to-even, then packs and stores; the integer-only requantization
//     is evaluated exactly (see epi_store16).
//
// qconv_pipe (8-bit activations, C_in % 64 == 0): a 4-deep ring of LDS stages
//   filled by global_load_lds_dwordx4 (global -> LDS without registers).  The
//   uint8 shift is applied to the fragments after they are read from LDS, and
//   out-of-image taps / rows past the end load a 16-byte row of pad codes kept in
//   the packed layer, so the DMA needs no per-element work.  LDS rows are 64 bytes
//   with their four 16-byte slots XOR-swizzled, which keeps both the DMA writes and
//   the 16-byte fragment reads free of bank conflicts.
// qconv_igemm (every other case: 4-bit activations, C_in % 64 != 0, the 3-channel
//   stem): register-staged double buffering, transforms and padding applied while
//   staging, rows padded to 144 bytes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "iqnn_internal.h"

#pragma clang fp contract(off)

namespace iqnn {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

// BF6 (e3m2: sign, 3 exponent bits with bias 3, 2 mantissa bits) code of an integer in
// [-8, 8]; all of them are exact: 1 = 2^0, 3 = 2^1 * 1.5, 5 = 2^2 * 1.25, 7 = 2^2 * 1.75.
__device__ __forceinline__ uint32_t bf6_code(int v) {
    const int m = v < 0 ? -v : v;
    const uint32_t mag = m == 0 ? 0u : (m == 1 ? 12u : (m == 2 ? 16u : (m == 3 ? 18u : (m == 4 ? 20u :
                         (m == 5 ? 21u : (m == 6 ? 22u : (m == 7 ? 23u : 24u)))))));
    return (v < 0 ? 32u : 0u) | mag;
}
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) void* gbl_ptr_t;

constexpr int kLdsStride = kBK + 16;   // bytes per staged row (register-staged kernel)
constexpr int kSegPerRow = kBK / 16;   // 16-element segments per staged row (8)
constexpr int kRowsPerPass = 256 / kSegPerRow;

__device__ __forceinline__ uint32_t unpack_lo(uint32_t v, int sign) {
    uint32_t n = v & 0x0F0F0F0Fu;
    return sign ? (n | ((n & 0x08080808u) * 0x1Eu)) : n;
}
__device__ __forceinline__ uint32_t unpack_hi(uint32_t v, int sign) {
    uint32_t n = (v >> 4) & 0x0F0F0F0Fu;
    return sign ? (n | ((n & 0x08080808u) * 0x1Eu)) : n;
}

__device__ __forceinline__ int xcd_remap(int bid, int G) {
    const int xcd = bid & 7, idx = bid >> 3;
    const int q8 = G >> 3, r8 = G & 7;
    return (xcd < r8) ? xcd * (q8 + 1) + idx : r8 * (q8 + 1) + (xcd - r8) * q8 + idx;
}

// Tile of workgroup `bid`.  Logical ids are first made contiguous per XCD, then
// walked in groups of `group_px` pixel tiles: inside a group, channel tiles are the
// outer loop and pixel tiles the inner one, so the workgroups that run together on
// one XCD share a few activation tiles and one weight tile, and that working set
// stays in the XCD's L2.
__device__ __forceinline__ void tile_of(int bid, int G, int n_oc, int n_px, int group_px, int& tile_oc,
                                        int& tile_px) {
    const int L = xcd_remap(bid, G);
    const int span = group_px * n_oc;
    const int pg = L / span;
    const int rem = L - pg * span;
    const int first = pg * group_px;
    const int gsize = min(group_px, n_px - first);
    tile_oc = rem / gsize;
    tile_px = first + (rem - tile_oc * gsize);
}

// Per-lane channel parameters for 16 consecutive channels starting at ocb.
struct ChanParams {
    int32_t bias[16];
    float mult[16];
};

__device__ __forceinline__ void load_chan(const ConvParams& p, int ocb, ChanParams& c) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        int4 bv = *reinterpret_cast<const int4*>(p.bias + ocb + 4 * j);
        float4 mv = *reinterpret_cast<const float4*>(p.mult + ocb + 4 * j);
        c.bias[4 * j] = bv.x; c.bias[4 * j + 1] = bv.y; c.bias[4 * j + 2] = bv.z; c.bias[4 * j + 3] = bv.w;
        c.mult[4 * j] = mv.x; c.mult[4 * j + 1] = mv.y; c.mult[4 * j + 2] = mv.z; c.mult[4 * j + 3] = mv.w;
    }
}

// Residual words of 16 consecutive channels (8-bit: 4 words; 4-bit: 2 words).
__device__ __forceinline__ void load_res16(const ConvParams& p, int64_t oidx, int ocb, uint32_t rw[4]) {
    rw[0] = rw[1] = rw[2] = rw[3] = 0;
    if (p.res_type == T_INT8 || p.res_type == T_UINT8) {
        if (p.vec_store) {
            uint4 v = *reinterpret_cast<const uint4*>(p.res + oidx);
            rw[0] = v.x; rw[1] = v.y; rw[2] = v.z; rw[3] = v.w;
        } else {
            for (int j = 0; j < 16 && ocb + j < p.c_out; ++j) rw[j >> 2] |= (uint32_t)p.res[oidx + j] << (8 * (j & 3));
        }
    } else {
        if (p.vec_store) {
            uint2 v = *reinterpret_cast<const uint2*>(p.res + (oidx >> 1));
            rw[0] = v.x; rw[1] = v.y;
        } else {
            for (int j = 0; j < 8 && ocb + 2 * j < p.c_out; ++j)
                rw[j >> 2] |= (uint32_t)p.res[(oidx >> 1) + j] << (8 * (j & 3));
        }
    }
}

// The clip / round / zero-point tail of the epilogue below: b[j] holds output code j
// in its low byte.
// FIX_LATER: the odd part of Z_out is left to the byte packer (pack_codes16).
__device__ __forceinline__ void round_codes16(const ConvParams& p, const float v[16], uint32_t b[16],
                                              bool fix_later = false) {
#pragma unroll
    for (int j = 0; j < 16; ++j)
        b[j] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_fmed3f(v[j], p.t_lo, p.t_hi) + p.out_magic);
    if (!fix_later && p.out_fix) {
#pragma unroll
        for (int j = 0; j < 16; ++j) b[j] += 1u;
    }
}

// The low bytes of b[0..15] as 16 consecutive bytes, plus the packed odd part of Z_out
// (p.out_fix4 = 0x01010101 when the host found that no byte can carry, see ConvParams).
__device__ __forceinline__ uint4 pack_bytes16(const ConvParams& p, const uint32_t b[16]) {
    uint32_t ow[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t lo2 = __builtin_amdgcn_perm(b[4 * d + 1], b[4 * d], 0x0C0C0400u);
        const uint32_t hi2 = __builtin_amdgcn_perm(b[4 * d + 3], b[4 * d + 2], 0x0C0C0400u);
        ow[d] = (lo2 | (hi2 << 16)) + p.out_fix4;
    }
    return make_uint4(ow[0], ow[1], ow[2], ow[3]);
}

// pack_bytes16 for codes rounded without the odd part of Z_out (round_codes16 with
// fix_later), adding it here: when a byte may hold 0xFF (p.out_fix = 1) each code is
// first placed in its own 16-bit lane, so adding 1 to every lane cannot carry into the
// next code, and a last permute keeps the low bytes -- five instructions per four codes
// instead of an addition per code.
__device__ __forceinline__ uint4 pack_codes16(const ConvParams& p, const uint32_t b[16]) {
    if (!p.out_fix) return pack_bytes16(p, b);
    uint32_t ow[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t lo2 = __builtin_amdgcn_perm(b[4 * d + 1], b[4 * d], 0x0C040C00u) + 0x00010001u;
        const uint32_t hi2 = __builtin_amdgcn_perm(b[4 * d + 3], b[4 * d + 2], 0x0C040C00u) + 0x00010001u;
        ow[d] = __builtin_amdgcn_perm(hi2, lo2, 0x06040200u);
    }
    return make_uint4(ow[0], ow[1], ow[2], ow[3]);
}

// Requantizing epilogue of 16 consecutive channels ocb..ocb+15 of output pixel pix,
// strict binary32 with one rounding per operation:
//   t = float(acc + bias) * M[c];   t = t + float(r - Z_res) * M_res   (ADD)
//   y = clip(rne(t) + Z_out, lo, Q_MAX)
// ReLU is the passive clamp at the real value 0 ("Quantization" blog, 量化激活函数):
// since rne is monotone and rne(0) = 0, clip(rne(max(t,0)) + Z) == clip(rne(t) + Z)
// with the lower bound raised to max(Q_MIN, Z_out).  The clip moves before the
// rounding, into the offset domain [lo - Z_out, hi - Z_out] (integer bounds, so
// rne(clip(t)) == clip(rne(t))).  Rounding and the zero point are one addition:
// C = 1.5 * 2^23 + Z_even, with Z_even the even part of Z_out, puts t + C in
// [2^23, 2^24) where binary32 steps by exactly 1, so the add rounds t to nearest
// even and the low mantissa bits hold rne(t) + Z_even (an even C keeps the tie
// parity of rne(t)).  Adding the odd part of Z_out (0 or 1) as an integer leaves the
// code in the low byte, two's complement for signed types; bytes are packed with
// v_perm_b32, nibbles with shifts.
//
// BIAS: add bias[] here (otherwise the accumulator started from the folded bias).
// ADDK: 0 = residual add decided by `add` and p.res_type at run time, 1 = always an
// 8-bit residual, 2 = never a residual, 3 = always a 4-bit residual.
// INTRQ: integer-only requantization (mult[] holds M_c * 2^-N_c, see below); compiled
// into the kernels' own integer-requantizing variants only.
// OUTK: 0 = output type and store width decided at run time; 1 = 8-bit codes, 2 = raw
// int32, 3 = 4-bit codes, each with 16-channel vector stores (C_out % 16 == 0).  A
// kernel that keeps most registers busy takes the one branch it needs.
// kept: with OUTK == 1, also receives the 16 stored bytes (a kernel that consumes its
// own output keeps them in LDS).
template <bool BIAS = true, int ADDK = 0, bool INTRQ = false, int OUTK = 0>
__device__ __forceinline__ void epi_store16(const ConvParams& p, const v16i& acc, const int32_t* bias,
                                            const float* mult, uint32_t rw[4], int ocb, int64_t pix, bool add_rt,
                                            float m_res, bool irq32 = false, uint4* kept = nullptr) {
    const bool add = (ADDK == 1 || ADDK == 3) ? true : (ADDK == 2 ? false : add_rt);
    const int64_t oidx = pix * p.c_out + ocb;   // element index of the first channel
    const bool vec = OUTK != 0 || p.vec_store;
    if (OUTK == 2 || (OUTK == 0 && p.epi == E_RAW)) {
        int32_t a[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) a[j] = acc[j] + (BIAS ? bias[j] : 0);
        int32_t* yo = reinterpret_cast<int32_t*>(p.y) + oidx;
        if (vec) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<int4*>(yo + 4 * j) = make_int4(a[4 * j], a[4 * j + 1], a[4 * j + 2], a[4 * j + 3]);
        } else {
            for (int j = 0; j < 16 && ocb + j < p.c_out; ++j) yo[j] = a[j];
        }
        return;
    }
    if constexpr (OUTK == 2) return;
    uint32_t b[16];
    if constexpr (INTRQ) {
        // integer-only requantization: mult[j] = x = M_c * 2^-N_c exactly (8-bit M_c),
        // and the code is clip(rne(a * M_c / 2^N_c)) + Z_out, rne half to even, with
        // a = acc + bias.  fma(float(a), x, 1.5 * 2^23) rounds once.  With |a| <= 2^24,
        // float(a) = a, and for |a x| < 2^22 the result is 1.5 * 2^23 + rne(a x), its
        // bits those of 1.5 * 2^23 plus the integer; a larger |a x| puts the result at
        // or beyond 2^24 (at or below 2^23), whose bits lie outside the clip range on
        // the same side: clipping the bits gives the exact code.  With |a| > 2^24 and
        // x >= 2^-13 (irq32: the caller checked every channel it stores), |a x| and
        // |float(a) x| exceed 2^11 with the same sign, and both clip to the same bound.
        // Otherwise such a lane takes binary64: a * M_c is below 2^40, so the product
        // and the scaling are exact and the one rounding of the fused add of 1.5 * 2^52
        // is the rne; the low word of the result is the integer.
        constexpr int32_t kB = 0x4B400000;   // bits of 1.5 * 2^23
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const float r = __builtin_fmaf((float)(acc[j] + (BIAS ? bias[j] : 0)), mult[j], 12582912.0f);
            b[j] = __builtin_bit_cast(uint32_t, r);
        }
        if (!irq32) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int32_t a = acc[j] + (BIAS ? bias[j] : 0);
                if (a > (1 << 24) || a < -(1 << 24)) {
                    // the multiplier's conversion stays in this rarely taken block (an
                    // ordinary conversion would be hoisted above it: 32 more registers
                    // and conversions on every tile)
                    double xd;
                    asm volatile("v_cvt_f64_f32 %0, %1" : "=v"(xd) : "v"(mult[j]));
                    const double r = __builtin_fma((double)a, xd, 6755399441055744.0);
                    const int32_t q = (int32_t)(uint32_t)__builtin_bit_cast(uint64_t, r);
                    b[j] = (uint32_t)(kB + min(max(q, -1024), 1024));
                }
            }
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int32_t q = min(max((int32_t)b[j], kB + p.q_lo), kB + p.q_hi);
            b[j] = (uint32_t)(q + (p.z_out - kB));
        }
    } else {
        float v[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) v[j] = (float)(acc[j] + (BIAS ? bias[j] : 0)) * mult[j];
        if (add) {
            const bool r8 = ADDK == 1 || (ADDK != 3 && (p.res_type == T_INT8 || p.res_type == T_UINT8));
            uint32_t w[4] = {rw[0] ^ p.res_xor, rw[1] ^ p.res_xor, rw[2] ^ p.res_xor, rw[3] ^ p.res_xor};
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const uint32_t code =
                    r8 ? (w[j >> 2] >> (8 * (j & 3))) & 0xFFu : (w[j >> 3] >> (4 * (j & 7))) & 0xFu;
                const float d = (float)code - p.res_zf;   // == float(r - Z_res), exact
                const float u = d * m_res;
                v[j] = v[j] + u;
            }
        }
        round_codes16(p, v, b, OUTK == 1);
    }
    if (OUTK == 1 || (OUTK == 0 && (p.y_type == T_INT8 || p.y_type == T_UINT8))) {
        const uint4 pk = (OUTK == 1 && !INTRQ) ? pack_codes16(p, b) : pack_bytes16(p, b);
        const uint32_t ow[4] = {pk.x, pk.y, pk.z, pk.w};
        if (vec) {
            *reinterpret_cast<uint4*>(p.y + oidx) = pk;
            if (OUTK == 1 && kept) *kept = pk;
        } else {
            for (int j = 0; j < 16 && ocb + j < p.c_out; ++j) p.y[oidx + j] = (uint8_t)(ow[j >> 2] >> (8 * (j & 3)));
        }
    } else {
        uint32_t ow[2] = {0, 0};
#pragma unroll
        for (int j = 0; j < 16; ++j) ow[j >> 3] |= (b[j] & 0xFu) << (4 * (j & 7));
        if (vec) {
            *reinterpret_cast<uint2*>(p.y + (oidx >> 1)) = make_uint2(ow[0], ow[1]);
        } else {
            for (int j = 0; j < 8 && ocb + 2 * j < p.c_out; ++j)
                p.y[(oidx >> 1) + j] = (uint8_t)(ow[j >> 2] >> (8 * (j & 3)));
        }
    }
}

// ============================================================ register-staged kernel

// The second launch bound is the number of workgroups per CU that the LDS
// footprint allows (160 KB of LDS per CU on gfx950).
template <int BM, int BN, int WM, int WN, int GATHER, bool IS1X1, bool INTRQ = false>
__global__ __launch_bounds__(256, (2 * 2 * (BM + BN) * kLdsStride <= 160 * 1024 ? 2 : 1))
void qconv_igemm(const ConvParams p) {
    constexpr int WPX = BN / WN;      // pixels per wave
    constexpr int TN = WPX / 32;      // 32x32 MFMA tiles along pixels per wave
    constexpr int TM = 2;             // 32x32 MFMA tiles along channels per wave (64 channels)
    constexpr int A_SEGS = BM * kSegPerRow / 256;
    constexpr int B_SEGS = BN * kSegPerRow / 256;
    static_assert(BM / WM == 64, "a wave owns 64 output channels");
    static_assert(WM * WN == 4, "four waves");
    static_assert(A_SEGS >= 1 && B_SEGS >= 1 && TN >= 1, "tile too small");

    __shared__ __attribute__((aligned(16))) uint8_t lds[2][(BM + BN) * kLdsStride];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wave_oc = wave % WM;
    const int wave_px = wave / WM;

    int tile_oc, tile_px;
    tile_of(blockIdx.x, gridDim.x, p.n_oc_tiles, p.n_px_tiles, p.group_px, tile_oc, tile_px);
    const int oc0 = tile_oc * BM;
    const int64_t px0 = (int64_t)tile_px * BN;

    // Staging assignment: thread -> (segment column, rows row0 + i*32).
    const int seg = tid % kSegPerRow;
    const int row0 = tid / kSegPerRow;

    // Per-row pixel geometry for the activation gather.
    int64_t rbase[B_SEGS];   // IS1X1: element offset of the pixel row; else of image n
    int32_t rih[B_SEGS], riw[B_SEGS];
#pragma unroll
    for (int i = 0; i < B_SEGS; ++i) {
        int64_t pix = px0 + row0 + i * kRowsPerPass;
        if (pix < p.m) {
            if (IS1X1) {
                rbase[i] = pix * p.c;
                rih[i] = 0;
                riw[i] = 0;
            } else {
                int64_t ohw = (int64_t)p.oh * p.ow;
                int64_t n = pix / ohw;
                int32_t rem = (int32_t)(pix - n * ohw);
                int32_t oy = rem / p.ow, ox = rem - oy * p.ow;
                rbase[i] = n * p.h * p.w_in * (int64_t)p.c;
                rih[i] = oy * p.sh - p.ph;
                riw[i] = ox * p.sw - p.pw;
            }
        } else {
            rbase[i] = -1;
            rih[i] = -(1 << 29);
            riw[i] = -(1 << 29);
        }
    }

    // K position of this thread's segment: k = ks + seg*16 at stage ks.
    // For the vector gathers a segment never straddles a tap (C % 16 == 0).
    int32_t kci = 0, kkx = 0, kky = 0;
    if (!IS1X1) {
        int32_t k = seg * 16;
        int32_t tap = k / p.c;
        kci = k - tap * p.c;
        kky = tap / p.kw;
        kkx = tap - kky * p.kw;
    }

    uint4 sa[A_SEGS];
    uint4 sb[B_SEGS];

    auto load_stage = [&](int k0) {
        // weights: rows oc0 + row, always inside the padded buffer
        const int kw_el = k0 + seg * 16;
#pragma unroll
        for (int i = 0; i < A_SEGS; ++i) {
            const int row = row0 + i * kRowsPerPass;
            if (kw_el < p.kp)
                sa[i] = *reinterpret_cast<const uint4*>(p.w + (int64_t)(oc0 + row) * p.kp + kw_el);
            else
                sa[i] = make_uint4(0, 0, 0, 0);
        }
        const bool kin = kw_el < p.k;
        if (GATHER == GATHER_B8 || GATHER == GATHER_B4) {
#pragma unroll
            for (int i = 0; i < B_SEGS; ++i) {
                bool ok;
                int64_t off;
                if (IS1X1) {
                    ok = kin && rbase[i] >= 0;
                    off = rbase[i] + kw_el;
                } else {
                    const int32_t iy = rih[i] + kky, ix = riw[i] + kkx;
                    ok = kin && (uint32_t)iy < (uint32_t)p.h && (uint32_t)ix < (uint32_t)p.w_in;
                    off = rbase[i] + ((int64_t)iy * p.w_in + ix) * p.c + kci;
                }
                if (GATHER == GATHER_B8) {
                    if (ok) {
                        uint4 v = *reinterpret_cast<const uint4*>(p.x + off);
                        v.x ^= p.x_xor; v.y ^= p.x_xor; v.z ^= p.x_xor; v.w ^= p.x_xor;
                        sb[i] = v;
                    } else {
                        sb[i] = make_uint4(p.pad_word, p.pad_word, p.pad_word, p.pad_word);
                    }
                } else {
                    if (ok) {
                        uint2 v = *reinterpret_cast<const uint2*>(p.x + (off >> 1));
                        sb[i] = make_uint4(unpack_lo(v.x, p.x_signed4), unpack_hi(v.x, p.x_signed4),
                                           unpack_lo(v.y, p.x_signed4), unpack_hi(v.y, p.x_signed4));
                    } else {
                        sb[i] = make_uint4(p.pad_word, p.pad_word, p.pad_word, p.pad_word);
                    }
                }
            }
        } else {
            // element gather: decode each of the 16 K positions
#pragma unroll
            for (int i = 0; i < B_SEGS; ++i) {
                uint32_t wv[4] = {0, 0, 0, 0};
                int32_t k = kw_el;
                int32_t tap = k / p.c;
                int32_t ci = k - tap * p.c;
                int32_t ky = tap / p.kw;
                int32_t kx = tap - ky * p.kw;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    uint32_t b = p.pad_word & 0xFF;
                    const int32_t iy = rih[i] + ky, ix = riw[i] + kx;
                    if (k + e < p.k && (uint32_t)iy < (uint32_t)p.h && (uint32_t)ix < (uint32_t)p.w_in) {
                        b = (p.x[rbase[i] + ((int64_t)iy * p.w_in + ix) * p.c + ci] ^ (p.x_xor & 0xFF));
                    }
                    wv[e >> 2] |= b << (8 * (e & 3));
                    if (++ci == p.c) {
                        ci = 0;
                        if (++kx == p.kw) { kx = 0; ++ky; }
                    }
                }
                sb[i] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
            }
        }
    };

    auto advance_k = [&]() {
        if (!IS1X1 && GATHER != GATHER_B8_ELEM) {
            kci += kBK;
            while (kci >= p.c) {
                kci -= p.c;
                if (++kkx == p.kw) { kkx = 0; ++kky; }
            }
        }
    };

    auto store_stage = [&](int buf) {
#pragma unroll
        for (int i = 0; i < A_SEGS; ++i) {
            const int row = row0 + i * kRowsPerPass;
            *reinterpret_cast<uint4*>(&lds[buf][row * kLdsStride + seg * 16]) = sa[i];
        }
#pragma unroll
        for (int i = 0; i < B_SEGS; ++i) {
            const int row = BM + row0 + i * kRowsPerPass;
            *reinterpret_cast<uint4*>(&lds[buf][row * kLdsStride + seg * 16]) = sb[i];
        }
    };

    v16i acc[TM][TN];
#pragma unroll
    for (int t = 0; t < TM; ++t)
#pragma unroll
        for (int u = 0; u < TN; ++u) acc[t][u] = v16i{};

    const int nstages = (p.kp + kBK - 1) / kBK;
    const int frag_row = lane & 31;
    const int frag_col = (lane >> 5) * 16;
    const int a_row0 = wave_oc * 64 + frag_row;
    const int b_row0 = BM + wave_px * WPX + frag_row;

    load_stage(0);
    advance_k();
    store_stage(0);
    __syncthreads();

    for (int s = 0; s < nstages; ++s) {
        const int buf = s & 1;
        const bool more = s + 1 < nstages;
        if (more) {
            load_stage((s + 1) * kBK);
            advance_k();
        }
        const uint8_t* L0 = lds[buf];
#pragma unroll
        for (int kk = 0; kk < kBK / 32; ++kk) {
            if (s * kBK + kk * 32 >= p.kp) break;
            v4i a[TM], b[TN];
#pragma unroll
            for (int t = 0; t < TM; ++t)
                a[t] = *reinterpret_cast<const v4i*>(&L0[(a_row0 + t * 32) * kLdsStride + kk * 32 + frag_col]);
#pragma unroll
            for (int u = 0; u < TN; ++u)
                b[u] = *reinterpret_cast<const v4i*>(&L0[(b_row0 + u * 32) * kLdsStride + kk * 32 + frag_col]);
#pragma unroll
            for (int t = 0; t < TM; ++t)
#pragma unroll
                for (int u = 0; u < TN; ++u)
                    acc[t][u] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[t], b[u], acc[t][u], 0, 0, 0);
        }
        if (more) store_stage(buf ^ 1);
        __syncthreads();
    }

    // ---------------------------------------------------------------- epilogue
    const bool add = p.epi == E_ADD || p.epi == E_ADD_RELU;
    const float m_res = add ? *p.m_res : 0.0f;
#pragma unroll
    for (int t = 0; t < TM; ++t) {
        const int ocb = oc0 + wave_oc * 64 + t * 32 + (lane >> 5) * 16;
        if (ocb >= p.c_out) continue;
        ChanParams cp;
        load_chan(p, ocb, cp);
#pragma unroll
        for (int u = 0; u < TN; ++u) {
            const int64_t pix = px0 + wave_px * WPX + u * 32 + frag_row;
            if (pix >= p.m) continue;
            uint32_t rw[4] = {0, 0, 0, 0};
            if (add) load_res16(p, pix * p.c_out + ocb, ocb, rw);
            epi_store16<true, 0, INTRQ>(p, acc[t][u], cp.bias, cp.mult, rw, ocb, pix, add, m_res);
        }
    }
}

// ============================================================ pipelined kernel

constexpr int kPipeBK = 64;     // K bytes per stage

// XOR swizzle of the four 16-byte slots of a 64-byte LDS row.  A fragment read is one
// ds_read_b128 of 32 consecutive rows x 2 slots; with the slot XORed by bits 2..3 of
// the row it runs conflict-free on gfx950 (measured: 4 LDS cycles per read, against
// 8 for the row>>1 family of swizzles and 16 unswizzled).
__device__ __forceinline__ int swz(int row) { return (row >> 2) & 3; }

// Swizzle of the 16-byte chunks of a residual row of `lpr` chunks (lpr = 2, 4, 8:
// 32-, 64-, 128-byte rows), chosen the same way: conflict-free reads of one chunk
// over 32 consecutive rows.
__device__ __forceinline__ int rswz(int row, int lpr) {
    return lpr == 8 ? (row >> 1) & 7 : (lpr == 4 ? (row >> 2) & 3 : (row >> 3) & 1);
}

// 4-bit activation rows in LDS are 32 bytes (64 codes) per stage; their two 16-byte
// halves are swapped on rows with bit 3 set (measured conflict-free for the
// 32-row x 2-half ds_read_b128).
__device__ __forceinline__ int swz4(int row) { return (row >> 3) & 1; }

// s_waitcnt for vmcnt <= n only (expcnt and lgkmcnt left at their maximum).
#define IQNN_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))
// s_waitcnt for vmcnt <= n and lgkmcnt == 0.
#define IQNN_WAIT_VM_LGKM0(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4))

// One tile configuration of the pipelined kernel: block BM channels x BN pixels,
// WM x (4/WM) waves, a ring of NST LDS stages.
template <int BM_, int BN_, int WM_, int NST_>
struct PipeCfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = 4 / WM_, NST = NST_;
    static constexpr int WOC = BM / WM;     // channels per wave
    static constexpr int WPX = BN / WN;     // pixels per wave
    static constexpr int TM = WOC / 32, TN = WPX / 32;
    static constexpr int STAGE = (BM + BN) * kPipeBK;
    // blocks per CU that the 160 KB of LDS allows (capped at 3: 168 VGPRs per lane)
    static constexpr int LDS_FIT = 160 * 1024 / (NST * STAGE);
    static constexpr int OCC = LDS_FIT >= 3 ? 3 : (LDS_FIT >= 2 ? 2 : 1);
    static_assert(STAGE >= 8 * BM, "epilogue tables live in ring slot 0");
};

// RES: 8-bit residual with C_out % 16 == 0, fetched into registers before the main
// loop so its latency hides behind the contraction.
// C4: the 4-channel gather (4-byte DMA per tap; see iqnn_api.cpp c4_path).
template <class C, bool IS1X1, bool RES, bool C4>
__global__ __launch_bounds__(256, C::OCC) void qconv_pipe(const ConvParams p) {
    constexpr int BM = C::BM, BN = C::BN, WM = C::WM, NST = C::NST;
    constexpr int TM = C::TM, TN = C::TN, STAGE = C::STAGE;
    constexpr int A_INST = BM / 64;   // DMA instructions (16 rows each) per wave per stage
    constexpr int B_INST = BN / 64;
    constexpr int LOADS = A_INST + (C4 ? BN / 16 : B_INST);
    static_assert(TM >= 1 && TN >= 1 && A_INST >= 1 && B_INST >= 1, "tile too small");
    static_assert(NST == 3 || NST == 4, "ring depth");

    // The ring is separate LDS arrays addressed with compile-time slot numbers, so the
    // compiler can tell the DMA into one slot from the fragment reads of another and
    // does not serialise them with a full vmcnt wait.
    __shared__ __attribute__((aligned(1024))) uint8_t lds0[STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t lds1[STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t lds2[STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t lds3[NST == 4 ? STAGE : 16];
    // the epilogue's per-channel bias and multiplier tables reuse ring slot 0 once the
    // contraction is done, so the whole LDS budget of a block is the ring
    int32_t* const cbias = reinterpret_cast<int32_t*>(lds0);
    float* const cmult = reinterpret_cast<float*>(lds0 + 4 * BM);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wave_oc = wave % WM;
    const int wave_px = wave / WM;

    int tile_oc, tile_px;
    tile_of(blockIdx.x, gridDim.x, p.n_oc_tiles, p.n_px_tiles, p.group_px, tile_oc, tile_px);
    const int oc0 = tile_oc * BM;
    const int64_t px0 = (int64_t)tile_px * BN;

    // channel parameters of this block (the packed arrays are padded past oc0 + BM)
    int32_t my_bias = 0;
    float my_mult = 0.0f;
    if (tid < BM) {
        my_bias = p.bias[oc0 + tid];
        my_mult = p.mult[oc0 + tid];
    }

    // DMA lane assignment: instruction j of this wave fills 16 LDS rows; lane -> row
    // (lane / 4), slot (lane % 4), which holds global K segment slot ^ swz(row).
    const int drow = lane >> 2;
    const int dslot = lane & 3;
    const uint8_t* padrow = p.pad_row;

    const int8_t* wsrc[A_INST];
#pragma unroll
    for (int j = 0; j < A_INST; ++j) {
        const int row = wave * (BM / 4) + 16 * j + drow;
        wsrc[j] = p.w + (int64_t)(oc0 + row) * p.kp + (dslot ^ swz(row)) * 16;
    }
    int64_t rbase[B_INST];
    int32_t rih[B_INST], riw[B_INST];
    int32_t bseg[B_INST];
#pragma unroll
    for (int j = 0; j < B_INST; ++j) {
        const int row = wave * (BN / 4) + 16 * j + drow;
        bseg[j] = (dslot ^ swz(row)) * 16;
        const int64_t pix = px0 + row;
        if (pix < p.m) {
            if (IS1X1) {
                rbase[j] = pix * p.c;
                rih[j] = 0;
                riw[j] = 0;
            } else {
                const int64_t ohw = (int64_t)p.oh * p.ow;
                const int64_t n = pix / ohw;
                const int32_t rem = (int32_t)(pix - n * ohw);
                const int32_t oy = rem / p.ow, ox = rem - oy * p.ow;
                rbase[j] = n * p.h * p.w_in * (int64_t)p.c;
                rih[j] = oy * p.sh - p.ph;
                riw[j] = ox * p.sw - p.pw;
            }
        } else {
            rbase[j] = -1;
            rih[j] = -(1 << 29);
            riw[j] = -(1 << 29);
        }
    }

    // 4-channel gather: each 4-byte DMA instruction fills 4 rows; lane -> row
    // (lane / 16), 4-byte position (lane % 16) = tap j of slot s, holding K segment
    // s ^ swz(row) of that row.
    // With the filter row widened to KWP in {4, 8, 16} taps, a 64-element stage is 16
    // taps = 16 / KWP whole filter rows, so a lane's tap column is the same in every
    // stage and its filter row advances by 16 / KWP per stage.
    constexpr int C4_INST = C4 ? BN / 16 : 1;
    int32_t coff[C4_INST];    // input pixel index of this lane's tap at stage 0 (-1: row past the end)
    int32_t cky[C4_INST];     // its filter row at stage 0
    if constexpr (C4) {
#pragma unroll
        for (int j = 0; j < C4_INST; ++j) {
            const int row = wave * (BN / 4) + 4 * j + (lane >> 4);
            const int slot = (lane >> 2) & 3, jj = lane & 3;
            const int tap0 = (slot ^ swz(row)) * 4 + jj;       // tap index inside the stage
            const int ky0 = tap0 / p.kw, kx0 = tap0 - ky0 * p.kw;
            const int64_t pix = px0 + row;
            coff[j] = -1;
            cky[j] = ky0;
            if (pix < p.m) {
                const int64_t ohw = (int64_t)p.oh * p.ow;
                const int32_t n = (int32_t)(pix / ohw);
                const int32_t rem = (int32_t)(pix - (int64_t)n * ohw);
                const int32_t oy = rem / p.ow, ox = rem - oy * p.ow;
                coff[j] = (n * p.h + oy * p.sh + ky0) * p.w_in + ox * p.sw + kx0;
            }
        }
    }

    const int nst = p.kp / kPipeBK;   // K % 64 == 0 on this path

    // Issue the DMA of stage s into ring slot `dst`.  With C % 64 == 0 a 64-element K
    // chunk lies inside one filter tap, so the tap is wave-uniform.
    auto issue = [&](int s, uint8_t* dst) {
        const int k0 = s * kPipeBK;
#pragma unroll
        for (int j = 0; j < A_INST; ++j) {
            uint8_t* d = dst + (wave * (BM / 4) + 16 * j) * kPipeBK;
            __builtin_amdgcn_global_load_lds((gbl_ptr_t)(wsrc[j] + k0), (lds_ptr_t)d, 16, 0, 0);
        }
        if constexpr (C4) {
#pragma unroll
            for (int j = 0; j < C4_INST; ++j) {
                uint8_t* d = dst + (BM + wave * (BN / 4) + 4 * j) * kPipeBK;
                const int32_t rows = s * (16 / p.kw);   // filter rows advanced since stage 0
                const uint8_t* src = padrow;
                if (coff[j] >= 0 && cky[j] + rows < p.kh)
                    src = p.x + (int64_t)(coff[j] + rows * p.w_in) * 4;
                __builtin_amdgcn_global_load_lds((gbl_ptr_t)src, (lds_ptr_t)d, 4, 0, 0);
            }
            return;
        }
        int32_t ci0 = k0, ky = 0, kx = 0;
        if (!IS1X1) {
            const int32_t tap = k0 / p.c;
            ci0 = k0 - tap * p.c;
            ky = tap / p.kw;
            kx = tap - ky * p.kw;
        }
#pragma unroll
        for (int j = 0; j < B_INST; ++j) {
            uint8_t* d = dst + (BM + wave * (BN / 4) + 16 * j) * kPipeBK;
            const uint8_t* src;
            if (IS1X1) {
                src = rbase[j] >= 0 ? p.x + rbase[j] + k0 + bseg[j] : padrow;
            } else {
                const int32_t iy = rih[j] + ky, ix = riw[j] + kx;
                const bool ok = (uint32_t)iy < (uint32_t)p.h && (uint32_t)ix < (uint32_t)p.w_in;
                src = ok ? p.x + rbase[j] + ((int64_t)iy * p.w_in + ix) * p.c + ci0 + bseg[j] : padrow;
            }
            __builtin_amdgcn_global_load_lds((gbl_ptr_t)src, (lds_ptr_t)d, 16, 0, 0);
        }
    };

    constexpr int D = NST - 1;   // prefetch distance in stages
    issue(0, lds0);
    if (nst > 1) issue(1, lds1);
    if (D > 2 && nst > 2) issue(2, lds2);

    // residual fragments for the epilogue, fetched now
    const int frow = lane & 31;
    uint4 rres[TM][TN];
    if (RES) {
#pragma unroll
        for (int t = 0; t < TM; ++t)
#pragma unroll
            for (int u = 0; u < TN; ++u) {
                const int ocb = oc0 + wave_oc * C::WOC + t * 32 + (lane >> 5) * 16;
                const int64_t pix = px0 + wave_px * C::WPX + u * 32 + frow;
                rres[t][u] = make_uint4(0, 0, 0, 0);
                if (ocb < p.c_out && pix < p.m)
                    rres[t][u] = *reinterpret_cast<const uint4*>(p.res + pix * p.c_out + ocb);
            }
    }
    v16i acc[TM][TN];
#pragma unroll
    for (int t = 0; t < TM; ++t)
#pragma unroll
        for (int u = 0; u < TN; ++u) acc[t][u] = v16i{};

    // fragment offsets inside a stage: row lane%32 of each tile, K slot per k-step
    const int fsw = swz(frow);
    const int foff0 = frow * kPipeBK + (((lane >> 5) + 0) ^ fsw) * 16;
    const int foff1 = frow * kPipeBK + (((lane >> 5) + 2) ^ fsw) * 16;
    const uint32_t bxor = p.x_xor;

    // Software pipeline per stage (two k-steps of 32):
    //   1. k-step-0 MFMAs, with the k-step-1 fragment reads slotted one by one between
    //      them (pinned by sched_group_barrier), so LDS latency hides behind the matrix pipe;
    //   2. k-step-1 MFMAs, issued before the next stage's barrier so the wait at the
    //      barrier overlaps matrix work;
    //   3. the next stage's barrier and refill DMA, then its k-step-0 fragment reads.
    v4i fa0[TM], fb0[TN], fa1[TM], fb1[TN];
    auto read_frags = [&](const uint8_t* cur, int fo, v4i (&fa)[TM], v4i (&fb)[TN]) {
#pragma unroll
        for (int t = 0; t < TM; ++t)
            fa[t] = *reinterpret_cast<const v4i*>(cur + (wave_oc * C::WOC + 32 * t) * kPipeBK + fo);
#pragma unroll
        for (int u = 0; u < TN; ++u)
            fb[u] = *reinterpret_cast<const v4i*>(cur + (BM + wave_px * C::WPX + 32 * u) * kPipeBK + fo);
    };
    auto shift_b = [&](v4i (&fb)[TN]) {
#pragma unroll
        for (int u = 0; u < TN; ++u) {
            fb[u][0] ^= bxor; fb[u][1] ^= bxor; fb[u][2] ^= bxor; fb[u][3] ^= bxor;
        }
    };
    // MFMAs number i in [lo, hi) of the TM x TN fragment grid, row-major
    auto mfmas = [&](v4i (&fa)[TM], v4i (&fb)[TN], int lo, int hi) {
#pragma unroll
        for (int t = 0; t < TM; ++t)
#pragma unroll
            for (int u = 0; u < TN; ++u)
                if (t * TN + u >= lo && t * TN + u < hi)
                    acc[t][u] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[t], fb[u], acc[t][u], 0, 0, 0);
    };
    // Stage s is ready once this wave's DMA for it has landed (vmcnt) and every wave
    // has passed the barrier.  lgkmcnt(0) first: this wave's reads of the slot about to
    // be refilled must be complete before anyone passes.  Plain s_barrier, not
    // __syncthreads(): its fence would wait for every DMA in flight and collapse the
    // ring.  After the barrier the slot freed by stage s-1 is refilled with stage s+D.
    auto sync_stage = [&](int s, uint8_t* refill) {
        const int ahead = nst - 1 - s;
        if (D - 1 >= 2 && ahead >= 2) IQNN_WAIT_VM_LGKM0(2 * LOADS);
        else if (ahead >= 1) IQNN_WAIT_VM_LGKM0(LOADS);
        else IQNN_WAIT_VM_LGKM0(0);
        __builtin_amdgcn_s_barrier();
        if (s + D < nst) issue(s + D, refill);
    };
    constexpr int NMF = TM * TN, NRD = TM + TN, HALF = NMF / 2;
    auto stage = [&](int s, const uint8_t* cur, const uint8_t* next, uint8_t* next_refill) {
        shift_b(fb0);
        __builtin_amdgcn_sched_barrier(0);
        mfmas(fa0, fb0, 0, NMF);
        read_frags(cur, foff1, fa1, fb1);
        // interleave: MFMA, read, MFMA, read, ... then the remaining MFMAs
#pragma unroll
        for (int i = 0; i < (NMF < NRD ? NMF : NRD); ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
        }
        if (NMF > NRD) __builtin_amdgcn_sched_group_barrier(0x008, NMF - NRD, 0);
        if (NRD > NMF) __builtin_amdgcn_sched_group_barrier(0x100, NRD - NMF, 0);
        __builtin_amdgcn_sched_barrier(0);
        shift_b(fb1);
        mfmas(fa1, fb1, 0, HALF);
        __builtin_amdgcn_sched_barrier(0);
        if (s + 1 < nst) sync_stage(s + 1, next_refill);
        // the next stage's k-step-0 reads go out first and land behind the other half of
        // the k-step-1 MFMAs.  Unconditional, so the wait-count pass keeps them ordered;
        // after the last stage they re-read valid LDS and the values are unused.
        read_frags(next, foff0, fa0, fb0);
        mfmas(fa1, fb1, HALF, NMF);
        __builtin_amdgcn_sched_group_barrier(0x100, NRD, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, NMF - HALF, 0);
        __builtin_amdgcn_sched_barrier(0);
    };

    sync_stage(0, NST == 4 ? lds3 : lds2);
    read_frags(lds0, foff0, fa0, fb0);
    if constexpr (NST == 4) {
        for (int s = 0; s < nst; s += 4) {
            stage(s, lds0, lds1, lds0);
            if (s + 1 < nst) stage(s + 1, lds1, lds2, lds1);
            if (s + 2 < nst) stage(s + 2, lds2, lds3, lds2);
            if (s + 3 < nst) stage(s + 3, lds3, lds0, lds3);
        }
    } else {
        for (int s = 0; s < nst; s += 3) {
            stage(s, lds0, lds1, lds0);
            if (s + 1 < nst) stage(s + 1, lds1, lds2, lds1);
            if (s + 2 < nst) stage(s + 2, lds2, lds0, lds2);
        }
    }

    // ---------------------------------------------------------------- epilogue
    __syncthreads();   // every wave is done with the ring
    if (tid < BM) {
        cbias[tid] = my_bias;
        cmult[tid] = my_mult;
    }
    __syncthreads();
    const bool add = p.epi == E_ADD || p.epi == E_ADD_RELU;
    const float m_res = add ? *p.m_res : 0.0f;
#pragma unroll
    for (int t = 0; t < TM; ++t) {
        const int ocl = wave_oc * C::WOC + t * 32 + (lane >> 5) * 16;   // channel inside the block
        const int ocb = oc0 + ocl;
        if (ocb >= p.c_out) continue;
        ChanParams cp;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int4 bv = *reinterpret_cast<const int4*>(&cbias[ocl + 4 * j]);
            float4 mv = *reinterpret_cast<const float4*>(&cmult[ocl + 4 * j]);
            cp.bias[4 * j] = bv.x; cp.bias[4 * j + 1] = bv.y; cp.bias[4 * j + 2] = bv.z; cp.bias[4 * j + 3] = bv.w;
            cp.mult[4 * j] = mv.x; cp.mult[4 * j + 1] = mv.y; cp.mult[4 * j + 2] = mv.z; cp.mult[4 * j + 3] = mv.w;
        }
#pragma unroll
        for (int u = 0; u < TN; ++u) {
            const int64_t pix = px0 + wave_px * C::WPX + u * 32 + frow;
            if (pix >= p.m) continue;
            uint32_t rw[4] = {0, 0, 0, 0};
            if (RES) {
                rw[0] = rres[t][u].x; rw[1] = rres[t][u].y; rw[2] = rres[t][u].z; rw[3] = rres[t][u].w;
            } else if (add) {
                load_res16(p, pix * p.c_out + ocb, ocb, rw);
            }
            epi_store16(p, acc[t][u], cp.bias, cp.mult, rw, ocb, pix, add, m_res);
        }
    }
}

// Pixel tiles per rasterization group: about 1.5 MB of activation tiles (the
// gathered tile bytes are BN * K), and at most an eighth of all pixel tiles so every
// XCD gets its own groups.
int group_px_for(int64_t n_px, int64_t tile_bytes) {
    int64_t g = (int64_t)(1536 * 1024) / (tile_bytes > 0 ? tile_bytes : 1);
    const int64_t eighth = (n_px + 7) / 8;
    if (g > eighth) g = eighth;
    if (g < 1) g = 1;
    return (int)g;
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_staged(const ConvParams& p, int gather, bool is_1x1, hipStream_t stream) {
    ConvParams q = p;
    q.n_oc_tiles = (p.c_out + BM - 1) / BM;
    const int64_t n_px = (p.m + BN - 1) / BN;
    const int64_t grid = n_px * q.n_oc_tiles;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
    q.n_px_tiles = (int32_t)n_px;
    q.group_px = group_px_for(n_px, (int64_t)BN * p.k);
    dim3 g((unsigned)grid), b(256);
    if (p.int_rq) {   // integer-only requantization: its own instantiations
        if (gather == GATHER_B8 && is_1x1)
            hipLaunchKernelGGL((qconv_igemm<BM, BN, WM, WN, GATHER_B8, true, true>), g, b, 0, stream, q);
        else if (gather == GATHER_B8)
            hipLaunchKernelGGL((qconv_igemm<BM, BN, WM, WN, GATHER_B8, false, true>), g, b, 0, stream, q);
        else if (gather == GATHER_B4 && is_1x1)
            hipLaunchKernelGGL((qconv_igemm<BM, BN, WM, WN, GATHER_B4, true, true>), g, b, 0, stream, q);
        else if (gather == GATHER_B4)
            hipLaunchKernelGGL((qconv_igemm<BM, BN, WM, WN, GATHER_B4, false, true>), g, b, 0, stream, q);
        else if (gather == GATHER_B8_ELEM)
            hipLaunchKernelGGL((qconv_igemm<BM, BN, WM, WN, GATHER_B8_ELEM, false, true>), g, b, 0, stream, q);
        else
            return hipErrorInvalidValue;
        return hipGetLastError();
    }
    if (gather == GATHER_B8 && is_1x1)
        hipLaunchKernelGGL((qconv_igemm<BM, BN, WM, WN, GATHER_B8, true>), g, b, 0, stream, q);
    else if (gather == GATHER_B8)
        hipLaunchKernelGGL((qconv_igemm<BM, BN, WM, WN, GATHER_B8, false>), g, b, 0, stream, q);
    else if (gather == GATHER_B4 && is_1x1)
        hipLaunchKernelGGL((qconv_igemm<BM, BN, WM, WN, GATHER_B4, true>), g, b, 0, stream, q);
    else if (gather == GATHER_B4)
        hipLaunchKernelGGL((qconv_igemm<BM, BN, WM, WN, GATHER_B4, false>), g, b, 0, stream, q);
    else
        hipLaunchKernelGGL((qconv_igemm<BM, BN, WM, WN, GATHER_B8_ELEM, false>), g, b, 0, stream, q);
    return hipGetLastError();
}

template <class C>
hipError_t launch_pipe(const ConvParams& p, bool is_1x1, bool res_prefetch, bool c4, hipStream_t stream) {
    ConvParams q = p;
    q.n_oc_tiles = (p.c_out + C::BM - 1) / C::BM;
    const int64_t n_px = (p.m + C::BN - 1) / C::BN;
    const int64_t grid = n_px * q.n_oc_tiles;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
    q.n_px_tiles = (int32_t)n_px;
    q.group_px = group_px_for(n_px, (int64_t)C::BN * p.k);
    dim3 g((unsigned)grid), b(256);
    if constexpr (C::BM <= 128 && C::BN <= 256 && C::NST == 4) {   // the 4-channel gather's shapes
        if (c4 && res_prefetch) {
            hipLaunchKernelGGL((qconv_pipe<C, false, true, true>), g, b, 0, stream, q);
            return hipGetLastError();
        }
        if (c4) {
            hipLaunchKernelGGL((qconv_pipe<C, false, false, true>), g, b, 0, stream, q);
            return hipGetLastError();
        }
    } else if (c4) {
        return hipErrorInvalidValue;
    }
    if (is_1x1 && res_prefetch)
        hipLaunchKernelGGL((qconv_pipe<C, true, true, false>), g, b, 0, stream, q);
    else if (is_1x1)
        hipLaunchKernelGGL((qconv_pipe<C, true, false, false>), g, b, 0, stream, q);
    else if (res_prefetch)
        hipLaunchKernelGGL((qconv_pipe<C, false, true, false>), g, b, 0, stream, q);
    else
        hipLaunchKernelGGL((qconv_pipe<C, false, false, false>), g, b, 0, stream, q);
    return hipGetLastError();
}

// ============================================================ streaming kernel
//
// qconv_stream: persistent workgroups that consume one continuous stream of LDS
// stages.  A workgroup keeps one channel tile for its whole life and walks a strided
// run of pixel tiles inside its XCD's contiguous share of the pixel range, so the
// channel tables are loaded once and the workgroups of an XCD that hold the other
// channel tiles read the same activation tiles at about the same time (one HBM read,
// the rest L2 hits).  The stream of a tile is its nst K-stages, then (Conv_Add_Relu
// with an 8-bit residual) one R-stage that brings the residual tile into LDS.  Stages
// are filled by LDS DMA NST-1 stages ahead, across tile boundaries, so the next
// tile's data is in flight while the epilogue of the current one runs and the ring
// never drains.
//
// The DMA is issued from inline assembly, invisible to the compiler's wait-count
// pass, so the ring can be one array addressed by a run-time slot without the
// compiler serialising every fragment read behind the DMA in flight.  Every wait on
// the ring is explicit: each issue is exactly K_LOADS DMA instructions per wave
// (R-stages are padded, the stream end re-issues its last stage into a free slot),
// so "stage g has landed" is always vmcnt <= (NST-2)*K_LOADS.  Loads return in
// order, so stores in flight can only make that wait stricter, never unsafe.

// LDS address (offset in the workgroup's LDS) of a __shared__ location
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(lds_ptr_t)(p);
}

// Runs of global -> LDS DMA issued from one m0 value.  Each instruction moves 16 (4)
// bytes per lane: lane i of instruction j writes LDS bytes [lds + j*STEP + 16 i, +16)
// ([lds + j*STEP + 4 i, +4)), STEP = 1024 (256).  The instruction's immediate offset
// shifts both the LDS and the global address (measured on gfx950), so each source
// pointer is passed lowered by j*STEP and m0 is written once per run.  m0 and its
// loads sit in one asm statement so nothing can use m0 in between; m0 takes one wait
// state before the first load reads it.  The LDS address is wave-uniform;
// readfirstlane pins it to an SGPR even when the compiler has parked it in a VGPR.
// One 16-byte-per-lane LDS DMA from a wave-uniform base address (SGPR pair) plus a
// per-lane unsigned 32-bit byte offset; the same m0 rules as dma16_run.
__device__ __forceinline__ void dma16_sbase(uint32_t lds, const void* sbase, uint32_t voff) {
    const uint32_t m = __builtin_amdgcn_readfirstlane(lds);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(m), "v"(voff), "s"(sbase)
                 : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void dma16_run(uint32_t lds, const void* const* src) {
    static_assert(N >= 1 && N <= 4, "16-byte runs of 1..4 KB");
    const uint32_t m = __builtin_amdgcn_readfirstlane(lds);
    const char* q0 = static_cast<const char*>(src[0]);
    if constexpr (N == 1) {
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m), "v"(q0)
                     : "memory", "m0");
    } else if constexpr (N == 2) {
        const char* q1 = static_cast<const char*>(src[1]) - 1024;
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\t"
                     "global_load_lds_dwordx4 %2, off offset:1024" ::"s"(m), "v"(q0), "v"(q1)
                     : "memory", "m0");
    } else if constexpr (N == 3) {
        const char* q1 = static_cast<const char*>(src[1]) - 1024;
        const char* q2 = static_cast<const char*>(src[2]) - 2048;
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\t"
                     "global_load_lds_dwordx4 %2, off offset:1024\n\tglobal_load_lds_dwordx4 %3, off offset:2048"
                     ::"s"(m), "v"(q0), "v"(q1), "v"(q2) : "memory", "m0");
    } else {
        const char* q1 = static_cast<const char*>(src[1]) - 1024;
        const char* q2 = static_cast<const char*>(src[2]) - 2048;
        const char* q3 = static_cast<const char*>(src[3]) - 3072;
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\t"
                     "global_load_lds_dwordx4 %2, off offset:1024\n\tglobal_load_lds_dwordx4 %3, off offset:2048\n\t"
                     "global_load_lds_dwordx4 %4, off offset:3072"
                     ::"s"(m), "v"(q0), "v"(q1), "v"(q2), "v"(q3) : "memory", "m0");
    }
}
// 16-byte DMA of N KB-instructions to consecutive KB of LDS, in runs of at most 4.
template <int N>
__device__ __forceinline__ void dma16_seq(uint32_t lds, const void* const* src) {
    if constexpr (N > 0) {
        constexpr int R = N < 4 ? N : 4;
        dma16_run<R>(lds, src);
        dma16_seq<N - R>(lds + R * 1024, src + R);
    }
}
// 4-byte DMA of N 256-byte instructions to consecutive LDS, in runs of 4.
template <int N>
__device__ __forceinline__ void dma4_seq(uint32_t lds, const void* const* src) {
    if constexpr (N > 0) {
        static_assert(N % 4 == 0, "4-byte runs of 4");
        const uint32_t m = __builtin_amdgcn_readfirstlane(lds);
        const char* q0 = static_cast<const char*>(src[0]);
        const char* q1 = static_cast<const char*>(src[1]) - 256;
        const char* q2 = static_cast<const char*>(src[2]) - 512;
        const char* q3 = static_cast<const char*>(src[3]) - 768;
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off\n\t"
                     "global_load_lds_dword %2, off offset:256\n\tglobal_load_lds_dword %3, off offset:512\n\t"
                     "global_load_lds_dword %4, off offset:768"
                     ::"s"(m), "v"(q0), "v"(q1), "v"(q2), "v"(q3) : "memory", "m0");
        dma4_seq<N - 4>(lds + 1024, src + 4);
    }
}

// 4-byte DMA of N = 1 or 2 256-byte instructions to consecutive LDS from one m0.
template <int N>
__device__ __forceinline__ void dma4_short(uint32_t lds, const void* const* src) {
    static_assert(N == 1 || N == 2, "short 4-byte runs");
    const uint32_t m = __builtin_amdgcn_readfirstlane(lds);
    const char* q0 = static_cast<const char*>(src[0]);
    if constexpr (N == 1) {
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off" ::"s"(m), "v"(q0)
                     : "memory", "m0");
    } else {
        const char* q1 = static_cast<const char*>(src[1]) - 256;
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off\n\t"
                     "global_load_lds_dword %2, off offset:256" ::"s"(m), "v"(q0), "v"(q1) : "memory", "m0");
    }
}

// OCC_: workgroups per CU to compile for (0: as many as the LDS allows, at most 2);
// 3 caps the kernel at 168 VGPRs.
// BROW_: bytes of an activation row per stage (32 for packed 4-bit activations).
// NW_: waves per workgroup, WM_ of them along channels.  Eight waves make one block
// per CU whose weight rows are fetched once for twice the pixels of a four-wave block,
// with two waves per SIMD as before.
template <int BM_, int BN_, int WM_, int NST_, int OCC_ = 0, int BROW_ = kPipeBK, int NW_ = 4>
struct StreamCfg {
    static constexpr int NW = NW_;
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = NW_ / WM_, NST = NST_;
    static constexpr int WOC = BM / WM, WPX = BN / WN;
    static constexpr int TM = WOC / 32, TN = WPX / 32;
    static constexpr int STAGE = BM * kPipeBK + BN * BROW_;
    static constexpr int LDS = NST * STAGE + 8 * BM;
    static constexpr int LDS_FIT = 160 * 1024 / LDS;   // 160 KB of LDS per CU
    static constexpr int OCC = OCC_ > 0 ? OCC_ : (LDS_FIT >= 2 && NW_ == 4 ? 2 : 1);
    static_assert(OCC <= LDS_FIT, "LDS for the requested occupancy");
    static_assert(WM * WN == NW && (NW == 4 || NW == 8), "four or eight waves");
};

// ZW: asymmetric weights.  The per-pixel sum of the activation operands is kept next
// to the contraction (one v_dot4 with ones per 16 bytes of a B fragment; lanes l and
// l+32 hold the two K halves of pixel l%32) and zw_red times it is added to every
// channel of the pixel before the epilogue.
// SP: 2:4 structured-sparse weights on the sparse MFMA (v_smfmac_i32_32x32x64_i8).  A
// stage's 64 K positions of a weight row are 32 bytes of kept codes (two per group of
// four K positions, in K order) and 8 bytes of 2-bit positions; lane half h of a
// 32-row fragment holds the kept codes of K [32h, 32h + 32) and their 16 positions
// (measured lane layout: kept code v pairs with B bytes 16h + 4*(v/2 % 4) + pos of
// B lane half v/8), and the B operand is the two 16-byte activation fragments the
// dense path reads for its two k-steps.  One sparse MFMA per stage replaces two.
// F6: 4-bit operands on the FP6 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4, both operands
// BF6 e3m2, unit scales): the INT4 weights come as BF6 codes from their own tile-order
// copy (64-byte LDS rows, 48 bytes used, 8-byte units swizzled by bits 2-4 of the row),
// the packed 4-bit activation rows are turned into BF6 per stage through a 256-entry
// table of code pairs (UINT4 codes shifted by -8, the shift folded into the bias), and
// one MFMA per stage accumulates in fp32, which is exact for these integers (a partial
// sum stays below 2^24); the epilogue converts it to int32 and adds the bias.
// OUTK: 1 = 8-bit output codes with 16-channel vector stores, fixed at compile time
// (the requantizing epilogue without run-time type branches); 4 = the same with the
// integer-only requantization; 0 = decided at run time.
// S4: 4-bit activations are INT4 (sign-extended when unpacked), else UINT4.
// W4: INT4 weights stay packed (two codes per byte, natural K order like an activation
// row) in the tile-order copy and in LDS: 32 bytes per weight row and stage.  A lane
// unpacks its A fragment by keeping each nibble in the high half of its byte -- the
// byte (w << 4) is the two's-complement int8 16*w, no sign extension needed -- so the
// contraction accumulates 16 * acc; the accumulators start from 16 * bias and are
// shifted right by 4 before the epilogue, which is exact (every term is a multiple
// of 16).
// f(integral_constant<int, 0>) ... f(integral_constant<int, N - 1>), unrolled
template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<N, I + 1>(f);
    }
}

// XS: the activation fragments take the uint8 sign flip (XOR with x_xor); false for
// signed 8-bit codes (x_xor == 0), whose fragments are MFMA operands as they are.
template <class C, bool IS1X1, bool RES, bool C4, bool B4 = false, bool ZW = false, bool SP = false,
          bool F6 = false, int OUTK = 0, bool S4 = false, bool W4 = false, bool XS = true, int SPL = 0>
__global__ __launch_bounds__(64 * C::NW, C::OCC) void qconv_stream(const ConvParams p) {
    constexpr int BM = C::BM, BN = C::BN, WM = C::WM, NST = C::NST, NW = C::NW;
    constexpr int TM = C::TM, TN = C::TN;
    constexpr int BROW = B4 ? 32 : kPipeBK;           // bytes of an activation row per stage
    constexpr int AROW = (SP || W4) ? 32 : kPipeBK;   // bytes of a weight row per stage (2:4: kept codes; packed INT4)
    constexpr int IROW = SP ? 8 : 0;                  // bytes of a weight row's sparse positions per stage
    constexpr int A_BYTES = BM * (AROW + IROW);       // weight part of a ring slot
    constexpr int RROW = B4 ? BM / 2 : BM;            // bytes of a residual row
    constexpr int STAGE_K = A_BYTES + BN * BROW;
    constexpr int STAGE = (RES && BN * RROW > STAGE_K) ? BN * RROW : STAGE_K;   // bytes of one ring slot
    // DMA instructions per wave per stage.  Weight rows: 32 (2:4) or 16 per instruction;
    // sparse positions: 32 rows per 4-byte instruction; activation rows: 16 (8-bit),
    // 32 (4-bit), 4 (4-channel gather) per instruction; residual: 1 KB per instruction
    constexpr int A_INST = SP ? BM / 128 : (W4 ? BM / (32 * NW) : BM / (16 * NW));
    constexpr int I_INST = SP ? BM / 128 : 0;
    constexpr int B_INST = C4 ? BN / (4 * NW) : (B4 ? BN / (32 * NW) : BN / (16 * NW));
    constexpr int K_LOADS = A_INST + I_INST + B_INST;
    constexpr int R_INST = RES ? BN * RROW / (1024 * NW) : 0;
    constexpr int D = NST - 1;                        // stages issued ahead
    static_assert(TM >= 1 && TN >= 1 && A_INST >= 1 && B_INST >= 1 && BN % 64 == 0, "tile shape");
    static_assert(C4 || SP || K_LOADS * 1024 * NW == STAGE, "a stage is K_LOADS KB-instructions per wave");
    static_assert(NW == 4 || !(SP || C4 || B4 || F6), "eight-wave blocks take the dense 8-bit gather");
    static_assert(BM <= 64 * NW, "one thread per channel loads the channel tables");
    static_assert(!SP || ((A_INST + B_INST) * 4096 + I_INST * 1024 == STAGE_K && BM % 128 == 0),
                  "a 2:4 stage: kept codes and activations in KB-instructions, positions in 256-byte ones");
    static_assert(!SP || !(B4 || C4 || ZW), "2:4 weights take the 8-bit gather with symmetric weights");
    static_assert(!(SP && RES) || NW * K_LOADS * 1024 <= STAGE, "the padded residual stage fits a slot");
    static_assert(!F6 || (B4 && !SP && !ZW && !C4), "the FP6 path takes packed 4-bit activations");
    static_assert(!W4 || (B4 && !F6 && A_INST * 32 * NW == BM), "packed INT4 weights: 4-bit streaming, whole KB");
    static_assert(!(B4 && C4), "one gather mode");
    static_assert(NST >= 3, "ring depth");
    static_assert(D * K_LOADS <= 60, "DMA in flight must fit the 6-bit vmcnt");
    static_assert(R_INST <= K_LOADS, "a residual tile fits one stage");
    static_assert(!(RES && C4), "the 4-channel gather has no residual stage");
    static_assert(!(ZW && (B4 || C4)), "the per-pixel weight zero-point term needs the 8-bit gather");
    static_assert(XS || !(B4 || SP || ZW || F6), "signed activations without the sign flip: the dense 8-bit path");
    static_assert(!RES || RROW == 32 || RROW == 64 || RROW == 128, "residual rows of 2, 4 or 8 chunks");

    __shared__ __attribute__((aligned(1024))) uint8_t ring[NST * STAGE];
    __shared__ __attribute__((aligned(16))) int32_t cbias[BM];
    __shared__ __attribute__((aligned(16))) float cmult[BM];
    __shared__ __attribute__((aligned(16))) uint32_t f6tab[F6 ? 256 : 1];   // byte -> BF6 code pair

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wave_oc = wave % WM;
    const int wave_px = wave / WM;

    // ------------------------------------------------------------ schedule
    // XCD x owns channel group x % xo_groups (n_oc of its channel tiles) and pixel share
    // x / xo_groups: with more than one channel group an XCD's weights stay in its L2
    const int xcd = blockIdx.x & 7, widx = blockIdx.x >> 3;
    const int n_oc = p.n_oc_tiles / p.xo_groups;
    const int oc_t = (xcd % p.xo_groups) * n_oc + widx % n_oc;
    const int member = widx / n_oc, members = p.gx / n_oc;
    const int chunk0 = (xcd / p.xo_groups) * p.px_chunk;
    const int chunk_len = min(p.px_chunk, p.n_px_tiles - chunk0);
    const int J = chunk_len > member ? (chunk_len - member + members - 1) / members : 0;
    if (J <= 0) return;
    const int oc0 = oc_t * BM;
    auto tile_px0 = [&](int j) -> int64_t { return (int64_t)(chunk0 + member + j * members) * BN; };

    if (tid < BM) {
        cbias[tid] = W4 ? p.bias[oc0 + tid] * 16 : p.bias[oc0 + tid];
        cmult[tid] = p.mult[oc0 + tid];
    }
    if constexpr (F6) {
        // the two codes of a byte: low nibble (even element) in bits 0-5, high in 6-11
        const int lo = tid & 15, hi = tid >> 4;
        const int vlo = p.x_signed4 ? (lo >= 8 ? lo - 16 : lo) : lo - 8;
        const int vhi = p.x_signed4 ? (hi >= 8 ? hi - 16 : hi) : hi - 8;
        f6tab[tid] = bf6_code(vlo) | (bf6_code(vhi) << 6);
    }
    __syncthreads();
    // integer-only requantization: the binary32 evaluation when every multiplier of the
    // wave's output channels is at least 2^-13 (a wave-uniform choice, see epi_store16)
    bool irq32 = false;
    if constexpr (OUTK == 4) {
        bool ok = true;
        for (int i = lane; i < C::WOC; i += 64) {
            const int c = wave_oc * C::WOC + i;
            ok = ok && (oc0 + c >= p.c_out || cmult[c] >= 0x1p-13f);
        }
        irq32 = __all(ok) != 0;
    }

    const int nst = p.kp / kPipeBK;
    constexpr int EXTRA = RES ? 1 : 0;
    const int spt = nst + EXTRA;   // stages per tile
    const uint32_t ring0 = lds_addr(ring);

    // ------------------------------------------------------------ issue side
    // DMA lane assignment of a K-stage: instruction j of this wave fills 16 LDS rows;
    // lane -> row lane/4, slot lane%4, which holds K segment slot ^ swz(row).
    const int drow = lane >> 2;
    const int dslot = lane & 3;
    const uint8_t* padrow = p.pad_row;
    const int8_t* wsrc[A_INST];
    const uint8_t* isrc[SP ? I_INST : 1];
#pragma unroll
    for (int j = 0; j < A_INST; ++j) {
        if constexpr (SP) {   // the block is the stage's LDS image: straight 1 KB copies
            wsrc[j] = p.w + (int64_t)oc_t * nst * kSpBlock + (wave * A_INST + j) * 1024 + lane * 16;
        } else if constexpr (W4) {   // 32 packed rows: one contiguous 1 KB piece of a 2 KB block
            const int row0 = oc0 + wave * (BM / NW) + 32 * j;
            wsrc[j] = p.w_tiled + ((int64_t)(row0 >> 6) * nst) * 2048 + (row0 & 63) * 32 + lane * 16;
        } else {   // 16 rows of the tile-order copy: one contiguous 1 KB piece of a 4 KB block
            const int row0 = oc0 + wave * (BM / NW) + 16 * j;
            wsrc[j] = p.w_tiled + ((int64_t)(row0 >> 6) * nst) * 4096 + (row0 & 63) * 64 + lane * 16;
        }
    }
    if constexpr (SP) {   // positions follow the kept codes in the block: 256-byte copies
        static_assert(!SP || BM == kSpRows, "2:4 blocks hold kSpRows channel rows");
#pragma unroll
        for (int j = 0; j < I_INST; ++j)
            isrc[j] = reinterpret_cast<const uint8_t*>(p.w) + (int64_t)oc_t * nst * kSpBlock + BM * AROW +
                      (wave * I_INST + j) * 256 + lane * 4;
    }
    // Per-tile state of the tile being issued.  Activation rows (B) are pixels:
    //   1x1:    prow = the pixel's row + its 16-byte segment; rows past the end point at
    //           the last pixel instead (a pixel's accumulator column depends only on its
    //           own row, and the epilogue never stores those columns), so a stage's
    //           address is prow + k0 with no test.
    //   KHxKW:  prow = the row of filter tap (0, 0), possibly outside the image, and
    //           tmask = the taps that fall inside it; a stage reads prow + tapoff when
    //           its tap is in tmask, else the row of pad codes.
    constexpr int NB = C4 ? 1 : B_INST;
    const uint8_t* prow[NB];
    // the split variant's layers have at most 32 filter taps (checked by the host)
    using MaskT = std::conditional_t<(SPL != 0), uint32_t, uint64_t>;
    MaskT tmask[NB];
    constexpr int C4N = C4 ? B_INST : 1;
    int32_t coff[C4N], cky[C4N];
    const uint8_t* rsrc[RES ? R_INST : 1];
    const uint32_t ohw = (uint32_t)(p.oh * p.ow);   // < 2^31, checked by the host
    auto set_issue_tile = [&](int j) {
        const int64_t px0 = tile_px0(j);
        if constexpr (C4) {
            // each 4-byte instruction fills 4 rows; lane -> row lane/16, 4-byte position
            // lane%16 = tap jj of slot s, holding K segment s ^ swz(row)
#pragma unroll
            for (int i = 0; i < B_INST; ++i) {
                const int row = wave * (BN / NW) + 4 * i + (lane >> 4);
                const int slot = (lane >> 2) & 3, jj = lane & 3;
                const int tap0 = (slot ^ swz(row)) * 4 + jj;
                const int ky0 = tap0 / p.kw, kx0 = tap0 - ky0 * p.kw;
                const int64_t pix = px0 + row;
                coff[i] = -1;
                cky[i] = ky0;
                if (pix < p.m) {
                    const uint32_t pu = (uint32_t)pix;
                    const uint32_t n = pu / ohw, rem = pu - n * ohw;
                    const uint32_t oy = rem / (uint32_t)p.ow, ox = rem - oy * (uint32_t)p.ow;
                    coff[i] = ((int32_t)n * p.h + (int32_t)oy * p.sh + ky0) * p.w_in + (int32_t)ox * p.sw + kx0;
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < B_INST; ++i) {
                // 8-bit: 16 rows of 64 bytes per instruction, lane -> row lane/4, slot lane%4;
                // 4-bit: 32 rows of 32 bytes, lane -> row lane/2, half lane%2
                const int row = B4 ? wave * (BN / NW) + 32 * i + (lane >> 1) : wave * (BN / NW) + 16 * i + drow;
                const int64_t pix = px0 + row;
                const int32_t seg = B4 ? ((lane & 1) ^ swz4(row)) * 16 : (dslot ^ swz(row)) * 16;
                constexpr int SH = B4 ? 1 : 0;   // element offset -> byte offset
                if (IS1X1) {
                    prow[i] = p.x + (((pix < p.m ? pix : p.m - 1) * p.c) >> SH) + seg;
                    tmask[i] = 0;
                } else if (pix < p.m) {
                    const uint32_t pu = (uint32_t)pix;
                    const uint32_t n = pu / ohw, rem = pu - n * ohw;
                    const uint32_t oy = rem / (uint32_t)p.ow, ox = rem - oy * (uint32_t)p.ow;
                    const int32_t iy0 = (int32_t)oy * p.sh - p.ph, ix0 = (int32_t)ox * p.sw - p.pw;
                    prow[i] = p.x + ((((int64_t)((int32_t)n * p.h + iy0) * p.w_in + ix0) * p.c) >> SH) + seg;
                    // taps inside the image: kx in [xlo, xhi), ky in [ylo, yhi)
                    const int32_t xlo = max(0, -ix0), xhi = min(p.kw, p.w_in - ix0);
                    const int32_t ylo = max(0, -iy0), yhi = min(p.kh, p.h - iy0);
                    uint64_t m = 0;
                    if (xlo < xhi) {
                        const uint64_t xm = ((uint64_t)1 << xhi) - ((uint64_t)1 << xlo);
                        for (int ky = ylo; ky < yhi; ++ky) m |= xm << (ky * p.kw);
                    }
                    tmask[i] = (MaskT)m;
                } else {
                    prow[i] = padrow;
                    tmask[i] = 0;
                }
            }
        }
        if constexpr (RES) {
            // residual rows [px][BM] bytes: instruction i of this wave covers 1024/BM rows,
            // BM/16 lanes per row
            constexpr int LPR = RROW / 16;
            constexpr int CPC = B4 ? 32 : 16;   // channels per 16-byte chunk
            constexpr int SH = B4 ? 1 : 0;
#pragma unroll
            for (int i = 0; i < R_INST; ++i) {
                const int row = (wave * R_INST + i) * (1024 / RROW) + lane / LPR;
                const int ch = oc0 + ((lane % LPR) ^ rswz(row, LPR)) * CPC;
                const int64_t pix = px0 + row;
                rsrc[i] = (pix < p.m && ch < p.c_out) ? p.res + ((pix * p.c_out + ch) >> SH) : p.res;
            }
        }
    };
    // the next stage to issue: local tile, stage in tile, ring slot, and its K position
    // (byte offset of the tap row plus channel offset from prow, tap index, channel
    // offset inside the tap, filter column)
    int is_j = 0, is_s = 0;
    uint32_t is_off = 0;
    int64_t tapoff = 0;
    int tap = 0, k_ci = 0, k_kx = 0;
    const int64_t row_jump = (int64_t)(p.w_in - p.kw) * p.c;   // end of a filter row -> start of the next
    set_issue_tile(0);
    // the pad row's address held in vector registers for the per-lane select (a select
    // cannot take it from scalar registers next to its condition)
    const uint8_t* padv = padrow;
    if constexpr (!IS1X1 && !C4) asm volatile("" : "+v"(padv));
    // SPLIT: KxK layers without a residual whose tiles have more than D + 1 stages.  The
    // issue side then reaches the next tile at a fixed stage of every tile, and the
    // stage loop is split there, so the per-tile rows and tap masks change only between
    // the two loops (no per-stage merge of them)
    static_assert(!SPL || (!IS1X1 && !C4 && !RES && !SP && !F6), "split stage loop: KxK gathers without a residual");
    constexpr bool split = SPL != 0;   // 2: also nst % NST == 0, the stages run in ring rounds
    bool frozen = false;   // split path: the issue side stays on the last stage of the last tile
    auto issue = [&](bool in_tile) {
        const uint32_t dst = ring0 + is_off;
        if (RES && is_s == nst) {
            if constexpr (RES) {
                const void* rs[R_INST];
#pragma unroll
                for (int i = 0; i < R_INST; ++i) rs[i] = rsrc[i];
                dma16_seq<R_INST>(dst + wave * R_INST * 1024, rs);
                constexpr int NPAD = K_LOADS - R_INST;   // padding: same count as a K-stage
                if constexpr (NPAD > 0) {
                    const void* ps[NPAD];
#pragma unroll
                    for (int i = 0; i < NPAD; ++i) ps[i] = p.res;
                    dma16_seq<NPAD>(dst + NW * R_INST * 1024 + wave * NPAD * 1024, ps);
                }
            }
        } else {
            const int k0 = is_s * kPipeBK;
            const void* as[A_INST];
#pragma unroll
            for (int j = 0; j < A_INST; ++j) as[j] = wsrc[j] + (int64_t)is_s * (SP ? kSpBlock : (W4 ? 2048 : 4096));
            dma16_seq<A_INST>(dst + wave * (BM / NW) * AROW, as);
            if constexpr (SP) {
                const void* is[I_INST];
#pragma unroll
                for (int j = 0; j < I_INST; ++j) is[j] = isrc[j] + (int64_t)is_s * kSpBlock;
                dma4_short<I_INST>(dst + BM * AROW + wave * (BM / NW) * IROW, is);
            }
            const void* bs[B_INST];
            if constexpr (C4) {
                const int32_t rows = is_s * (16 / p.kw);   // filter rows advanced since stage 0
#pragma unroll
                for (int i = 0; i < B_INST; ++i) {
                    const uint8_t* src = padrow;
                    if (coff[i] >= 0 && cky[i] + rows < p.kh) src = p.x + (int64_t)(coff[i] + rows * p.w_in) * 4;
                    bs[i] = src;
                }
                dma4_seq<B_INST>(dst + (BM + wave * (BN / NW)) * kPipeBK, bs);
            } else {
                constexpr int SH = B4 ? 1 : 0;
#pragma unroll
                for (int i = 0; i < B_INST; ++i) {
                    if constexpr (IS1X1) bs[i] = prow[i] + (k0 >> SH);
                    else bs[i] = ((tmask[i] >> tap) & 1) ? prow[i] + (tapoff >> SH) : padv;
                }
                dma16_seq<B_INST>(dst + A_BYTES + wave * (BN / NW) * BROW, bs);
            }
        }
        is_off = is_off + STAGE == NST * STAGE ? 0 : is_off + STAGE;
        // advance the cursor; past the end it stays on the last stage.  In the split
        // path the cursor never leaves its tile here (the loop switches it)
        if (in_tile) {
            if (!frozen && is_s + 1 < spt) {
                ++is_s;
                if (!IS1X1 && !C4 && is_s < nst) {
                    tapoff += kPipeBK;
                    k_ci += kPipeBK;
                    if (k_ci == p.c) {
                        k_ci = 0;
                        ++tap;
                        if (++k_kx == p.kw) {
                            k_kx = 0;
                            tapoff += row_jump;
                        }
                    }
                }
            }
        } else if (is_s + 1 < spt) {
            ++is_s;
            if (!IS1X1 && !C4 && is_s < nst) {
                tapoff += kPipeBK;
                k_ci += kPipeBK;
                if (k_ci == p.c) {
                    k_ci = 0;
                    ++tap;
                    if (++k_kx == p.kw) {
                        k_kx = 0;
                        tapoff += row_jump;
                    }
                }
            }
        } else if (is_j + 1 < J) {
            ++is_j;
            is_s = 0;
            tapoff = 0;
            tap = k_ci = k_kx = 0;
            set_issue_tile(is_j);
        }
    };

    // ------------------------------------------------------------ compute side
    const int frow = lane & 31;
    const int fsw = swz(frow);
    const int foff0 = frow * kPipeBK + (((lane >> 5) + 0) ^ fsw) * 16;
    const int foff1 = frow * kPipeBK + (((lane >> 5) + 2) ^ fsw) * 16;
    const uint32_t bxor = p.x_xor;
    // accumulators start from the folded bias of their channels: lane half h of channel
    // block t holds channels ocl(t) .. ocl(t)+15 of the block
    v16i acc[TM][TN];
    v16f accf[F6 ? TM : 1][F6 ? TN : 1];
    int32_t ssum[ZW ? TN : 1];
    auto init_acc = [&]() {
        if constexpr (F6) {
#pragma unroll
            for (int t = 0; t < TM; ++t)
#pragma unroll
                for (int u = 0; u < TN; ++u)
#pragma unroll
                    for (int q = 0; q < 16; ++q) accf[t][u][q] = 0.0f;
            return;
        }
        if constexpr (ZW) {
#pragma unroll
            for (int u = 0; u < TN; ++u) ssum[u] = 0;
        }
#pragma unroll
        for (int t = 0; t < TM; ++t) {
            const int ocl = wave_oc * C::WOC + t * 32 + (lane >> 5) * 16;
            v16i b;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int4 bv = *reinterpret_cast<const int4*>(&cbias[ocl + 4 * q]);
                b[4 * q] = bv.x; b[4 * q + 1] = bv.y; b[4 * q + 2] = bv.z; b[4 * q + 3] = bv.w;
            }
#pragma unroll
            for (int u = 0; u < TN; ++u) acc[t][u] = b;
        }
    };
    init_acc();

    v4i fa0[TM], fb0[TN], fa1[TM], fb1[TN];
    // 4-bit: a lane's 16 bytes of a pixel row hold its half of both k-steps (8 bytes
    // each), read once per stage at k-step 0 and unpacked per k-step
    uint4 b4raw[B4 ? TN : 1];
    // packed INT4 weights: a lane's 16 bytes of a weight row, both k-steps, likewise
    uint4 a4raw[W4 ? TM : 1];
    const int b4off = (((lane >> 5) ^ swz4(frow)) * 16) + frow * 32;
    constexpr int x_signed4 = S4 ? 1 : 0;
    auto read_frags = [&](const uint8_t* cur, int fo, v4i (&fa)[TM], v4i (&fb)[TN]) {
        if constexpr (W4) {
            if (fo == foff0) {
#pragma unroll
                for (int t = 0; t < TM; ++t)
                    a4raw[t] = *reinterpret_cast<const uint4*>(cur + (wave_oc * C::WOC + 32 * t) * 32 + b4off);
            }
        } else {
#pragma unroll
            for (int t = 0; t < TM; ++t)
                fa[t] = *reinterpret_cast<const v4i*>(cur + (wave_oc * C::WOC + 32 * t) * kPipeBK + fo);
        }
        if constexpr (B4) {
            if (fo == foff0) {
#pragma unroll
                for (int u = 0; u < TN; ++u)
                    b4raw[u] = *reinterpret_cast<const uint4*>(cur + A_BYTES + (wave_px * C::WPX + 32 * u) * 32 + b4off);
            }
        } else {
#pragma unroll
            for (int u = 0; u < TN; ++u)
                fb[u] = *reinterpret_cast<const v4i*>(cur + (BM + wave_px * C::WPX + 32 * u) * kPipeBK + fo);
        }
    };
    // the A fragments of k-step kk from packed INT4 weights: nibble j of each byte in
    // its high half, the int8 16*w (the same element order as the activation unpack)
    auto unpack_a = [&](v4i (&fa)[TM], int kk) {
        if constexpr (W4) {
#pragma unroll
            for (int t = 0; t < TM; ++t) {
                const uint32_t w0 = kk == 0 ? a4raw[t].x : a4raw[t].z, w1 = kk == 0 ? a4raw[t].y : a4raw[t].w;
                fa[t][0] = (int)((w0 << 4) & 0xF0F0F0F0u); fa[t][1] = (int)(w0 & 0xF0F0F0F0u);
                fa[t][2] = (int)((w1 << 4) & 0xF0F0F0F0u); fa[t][3] = (int)(w1 & 0xF0F0F0F0u);
            }
        }
    };
    // make the B fragments of k-step kk MFMA-ready: the uint8 shift (XOR 0x80), or the
    // 4-bit unpack (UINT4 zero-, INT4 sign-extended) of this k-step's 8 bytes
    auto shift_b = [&](v4i (&fb)[TN], int kk) {
#pragma unroll
        for (int u = 0; u < TN; ++u) {
            if constexpr (B4) {
                const uint32_t w0 = kk == 0 ? b4raw[u].x : b4raw[u].z, w1 = kk == 0 ? b4raw[u].y : b4raw[u].w;
                fb[u][0] = (int)unpack_lo(w0, x_signed4); fb[u][1] = (int)unpack_hi(w0, x_signed4);
                fb[u][2] = (int)unpack_lo(w1, x_signed4); fb[u][3] = (int)unpack_hi(w1, x_signed4);
            } else {
                if constexpr (XS) {
                    fb[u][0] ^= bxor; fb[u][1] ^= bxor; fb[u][2] ^= bxor; fb[u][3] ^= bxor;
                }
                if constexpr (ZW) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) ssum[u] = __builtin_amdgcn_sdot4(fb[u][i], 0x01010101, ssum[u], false);
                }
            }
        }
    };
    auto mfmas = [&](v4i (&fa)[TM], v4i (&fb)[TN], int lo, int hi) {
#pragma unroll
        for (int t = 0; t < TM; ++t)
#pragma unroll
            for (int u = 0; u < TN; ++u)
                if (t * TN + u >= lo && t * TN + u < hi)
                    acc[t][u] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[t], fb[u], acc[t][u], 0, 0, 0);
    };
    // The next stage is ready once this wave's DMA for it has landed and every wave has
    // passed the barrier; lgkmcnt(0) first, so the slot refilled right after the
    // barrier (the one consumed last) has no reads left in flight.
    auto sync = [&]() {
        IQNN_WAIT_VM_LGKM0((D - 1) * K_LOADS);
        __builtin_amdgcn_s_barrier();
        issue(split);
    };

    // 2:4 weights: the fragments of one stage (kept codes, positions, both activation
    // k-steps); two sets alternate so the next stage is read during this one's MFMAs
    struct SpFrag {
        v4i a[SP ? TM : 1];
        int ix[SP ? TM : 1];
        v4i b0[SP ? TN : 1], b1[SP ? TN : 1];
    };
    auto read_sp = [&](const uint8_t* cur, SpFrag& f) {
        if constexpr (SP) {
#pragma unroll
            for (int t = 0; t < TM; ++t) {
                const int row = wave_oc * C::WOC + 32 * t + frow;
                f.a[t] = *reinterpret_cast<const v4i*>(cur + row * AROW + (((lane >> 5) ^ swz4(row)) * 16));
                f.ix[t] = *reinterpret_cast<const int*>(cur + BM * AROW + row * IROW + (lane >> 5) * 4);
            }
#pragma unroll
            for (int u = 0; u < TN; ++u) {
                const uint8_t* brow = cur + A_BYTES + (wave_px * C::WPX + 32 * u) * kPipeBK;
                f.b0[u] = *reinterpret_cast<const v4i*>(brow + foff0);
                f.b1[u] = *reinterpret_cast<const v4i*>(brow + foff1);
            }
        }
    };
    auto smfmacs = [&](SpFrag& f, int lo, int hi) {
        if constexpr (SP) {
#pragma unroll
            for (int t = 0; t < TM; ++t)
#pragma unroll
                for (int u = 0; u < TN; ++u)
                    if (t * TN + u >= lo && t * TN + u < hi) {
                        const v8i b = {f.b0[u][0], f.b0[u][1], f.b0[u][2], f.b0[u][3],
                                       f.b1[u][0], f.b1[u][1], f.b1[u][2], f.b1[u][3]};
                        acc[t][u] = __builtin_amdgcn_smfmac_i32_32x32x64_i8(f.a[t], b, acc[t][u], f.ix[t], 0, 0);
                    }
        }
    };
    SpFrag fx, fy;

    // FP6 path: the fragments of one stage (BF6 weight codes, packed 4-bit activations)
    struct F6Frag {
        v8i a[F6 ? TM : 1];
        uint4 b[F6 ? TN : 1];
    };
    auto read_f6 = [&](const uint8_t* cur, F6Frag& f) {
        if constexpr (F6) {
#pragma unroll
            for (int t = 0; t < TM; ++t) {
                const int row = wave_oc * C::WOC + 32 * t + frow;
                const uint8_t* rp = cur + row * kPipeBK;
                const int sw = (row >> 2) & 7, u0 = 3 * (lane >> 5);
                const uint2 d0 = *reinterpret_cast<const uint2*>(rp + ((u0 ^ sw) << 3));
                const uint2 d1 = *reinterpret_cast<const uint2*>(rp + (((u0 + 1) ^ sw) << 3));
                const uint2 d2 = *reinterpret_cast<const uint2*>(rp + (((u0 + 2) ^ sw) << 3));
                f.a[t] = v8i{(int)d0.x, (int)d0.y, (int)d1.x, (int)d1.y, (int)d2.x, (int)d2.y, 0, 0};
            }
#pragma unroll
            for (int u = 0; u < TN; ++u)
                f.b[u] = *reinterpret_cast<const uint4*>(cur + A_BYTES + (wave_px * C::WPX + 32 * u) * 32 + b4off);
        }
    };
    // 32 packed 4-bit codes (16 bytes) -> 32 BF6 codes, code v at bits 6v..6v+5
    auto to_bf6 = [&](const uint4& raw) -> v8i {
        const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
        uint32_t pr[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) pr[q] = f6tab[(wd[q >> 2] >> (8 * (q & 3))) & 0xFFu];
        v8i o;
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            const uint32_t* P = pr + 8 * g;
            o[3 * g] = (int)(P[0] | (P[1] << 12) | (P[2] << 24));
            o[3 * g + 1] = (int)((P[2] >> 8) | (P[3] << 4) | (P[4] << 16) | (P[5] << 28));
            o[3 * g + 2] = (int)((P[5] >> 4) | (P[6] << 8) | (P[7] << 20));
        }
        o[6] = 0;
        o[7] = 0;
        return o;
    };
    F6Frag gx, gy;

    for (int i = 0; i < D; ++i) issue(split);
    uint32_t cur_off = 0;
    auto advance = [&]() { cur_off = cur_off + STAGE == NST * STAGE ? 0 : cur_off + STAGE; };
    sync();
    if constexpr (SP) read_sp(ring + cur_off, fx);
    else if constexpr (F6) read_f6(ring + cur_off, gx);
    else read_frags(ring + cur_off, foff0, fa0, fb0);

    constexpr int NMF = TM * TN, NRD = TM + TN, HALF = NMF / 2;
    // residual epilogues run only with the residual stage (the host routes the rest to
    // qconv_pipe), so no global load of the epilogue is ever pending in the loop
    constexpr bool add = RES;
    const float m_res = RES ? *p.m_res : 0.0f;
    // one 2:4 stage: the uint8 shift of its activation fragments, the first half of its
    // MFMAs, the stage barrier (and the DMA refill), the next stage's fragment reads
    // next to the second half
    auto sp_stage = [&](SpFrag& f, SpFrag& nf, bool more, bool do_sync) {
        if constexpr (SP) {
#pragma unroll
            for (int u = 0; u < TN; ++u)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    f.b0[u][i] ^= bxor;
                    f.b1[u][i] ^= bxor;
                }
            __builtin_amdgcn_sched_barrier(0);
            smfmacs(f, 0, HALF);
            __builtin_amdgcn_sched_barrier(0);
            advance();
            if (do_sync) sync();
            if (more) read_sp(ring + cur_off, nf);
            smfmacs(f, HALF, NMF);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // one FP6 stage: the activations to BF6, the first half of the MFMAs, the barrier
    // (and the DMA refill), the next stage's reads next to the second half
    auto f6_stage = [&](F6Frag& f, F6Frag& nf, bool more, bool do_sync) {
        if constexpr (F6) {
            v8i b6[TN];
#pragma unroll
            for (int u = 0; u < TN; ++u) b6[u] = to_bf6(f.b[u]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int t = 0; t < TM; ++t)
#pragma unroll
                for (int u = 0; u < TN; ++u)
                    if (t * TN + u < HALF)
                        accf[t][u] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.a[t], b6[u], accf[t][u], 3, 3,
                                                                                     0, 127, 0, 127);
            __builtin_amdgcn_sched_barrier(0);
            advance();
            if (do_sync) sync();
            if (more) read_f6(ring + cur_off, nf);
#pragma unroll
            for (int t = 0; t < TM; ++t)
#pragma unroll
                for (int u = 0; u < TN; ++u)
                    if (t * TN + u >= HALF)
                        accf[t][u] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.a[t], b6[u], accf[t][u], 3, 3,
                                                                                     0, 127, 0, 127);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // one stage of the dense path; slot_c: the stage's ring slot when known at compile
    // time (an integral constant), else -1 (the slot is read at run time)
    auto dense_stage_at = [&](auto slot_c, int s, bool last_tile) {
        constexpr int SLOT = decltype(slot_c)::value;
        const uint8_t* cur = SLOT >= 0 ? ring + SLOT * STAGE : ring + cur_off;
        shift_b(fb0, 0);
        unpack_a(fa0, 0);
        __builtin_amdgcn_sched_barrier(0);
        mfmas(fa0, fb0, 0, NMF);
        read_frags(cur, foff1, fa1, fb1);
#pragma unroll
        for (int i = 0; i < (NMF < NRD ? NMF : NRD); ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
        }
        if (NMF > NRD) __builtin_amdgcn_sched_group_barrier(0x008, NMF - NRD, 0);
        if (NRD > NMF) __builtin_amdgcn_sched_group_barrier(0x100, NRD - NMF, 0);
        __builtin_amdgcn_sched_barrier(0);
        shift_b(fb1, 1);
        unpack_a(fa1, 1);
        mfmas(fa1, fb1, 0, HALF);
        __builtin_amdgcn_sched_barrier(0);
        advance();
        if (!(last_tile && s + 1 == nst && !RES)) sync();
        if (s + 1 < nst)
            read_frags(SLOT >= 0 ? ring + ((SLOT + 1) % NST) * STAGE : ring + cur_off, foff0, fa0, fb0);
        mfmas(fa1, fb1, HALF, NMF);
        __builtin_amdgcn_sched_barrier(0);
    };
    // NST stages with their slots 0 .. NST-1 at compile time
    auto ring_round = [&](int s0, bool last_tile) {
        static_for<NST>([&](auto q) { dense_stage_at(q, s0 + decltype(q)::value, last_tile); });
    };

    for (int j = 0; j < J; ++j) {
        const bool last_tile = j + 1 == J;
        if constexpr (F6) {
            for (int s = 0; s < nst; s += 2) {
                const bool end0 = s + 1 == nst;
                f6_stage(gx, gy, !end0, !(last_tile && end0 && !RES));
                if (!end0) {
                    const bool end1 = s + 2 == nst;
                    f6_stage(gy, gx, !end1, !(last_tile && end1 && !RES));
                }
            }
        } else if constexpr (SP) {
            for (int s = 0; s < nst; s += 2) {
                const bool end0 = s + 1 == nst;
                sp_stage(fx, fy, !end0, !(last_tile && end0 && !RES));
                if (!end0) {
                    const bool end1 = s + 2 == nst;
                    sp_stage(fy, fx, !end1, !(last_tile && end1 && !RES));
                }
            }
        } else if constexpr (SPL == 1) {
            // the stage whose sync issues the next tile's first stage
            const int s_sw = nst - D - 1;
            for (int s = 0; s < s_sw; ++s) dense_stage_at(std::integral_constant<int, -1>{}, s, last_tile);
            if (!last_tile) {
                ++is_j;
                is_s = 0;
                tapoff = 0;
                tap = k_ci = k_kx = 0;
                set_issue_tile(is_j);
            } else {
                frozen = true;
            }
            for (int s = s_sw; s < nst; ++s) dense_stage_at(std::integral_constant<int, -1>{}, s, last_tile);
        } else if constexpr (SPL == 2) {
            // as above; nst is a multiple of NST (checked by the host), so every tile starts
            // in slot 0 and the slots of its stages are known in rounds of NST
            const int s_sw = nst - D - 1;
            for (int s = 0; s < s_sw; s += NST) ring_round(s, last_tile);
            if (!last_tile) {
                ++is_j;
                is_s = 0;
                tapoff = 0;
                tap = k_ci = k_kx = 0;
                set_issue_tile(is_j);
            } else {
                frozen = true;
            }
            ring_round(s_sw, last_tile);
        } else {
            for (int s = 0; s < nst; ++s) dense_stage_at(std::integral_constant<int, -1>{}, s, last_tile);
        }

        // -------------------------------------------------------- epilogue of tile j
        const int64_t px0 = tile_px0(j);
        const uint8_t* rtile = ring + cur_off;   // the R-stage, synced above
        if constexpr (ZW) {
#pragma unroll
            for (int u = 0; u < TN; ++u) {
                const int32_t red = p.zw_red * (ssum[u] + __shfl_xor(ssum[u], 32));
#pragma unroll
                for (int t = 0; t < TM; ++t)
#pragma unroll
                    for (int q = 0; q < 16; ++q) acc[t][u][q] += red;
            }
        }
#pragma unroll
        for (int t = 0; t < TM; ++t) {
            const int ocl = wave_oc * C::WOC + t * 32 + (lane >> 5) * 16;   // channel inside the block
            const int ocb = oc0 + ocl;
            if (ocb >= p.c_out) continue;
            float mult[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 mv = *reinterpret_cast<const float4*>(&cmult[ocl + 4 * q]);
                mult[4 * q] = mv.x; mult[4 * q + 1] = mv.y; mult[4 * q + 2] = mv.z; mult[4 * q + 3] = mv.w;
            }
#pragma unroll
            for (int u = 0; u < TN; ++u) {
                const int pl = wave_px * C::WPX + u * 32 + frow;   // pixel inside the block
                const int64_t pix = px0 + pl;
                if (pix >= p.m) continue;
                uint32_t rw[4] = {0, 0, 0, 0};
                if (RES && !B4) {
                    const uint4 v = *reinterpret_cast<const uint4*>(rtile + pl * RROW + (((ocl >> 4) ^ rswz(pl, RROW / 16)) << 4));
                    rw[0] = v.x; rw[1] = v.y; rw[2] = v.z; rw[3] = v.w;
                } else if (RES) {   // 16 channels = 8 bytes: half (ocl/16)%2 of chunk ocl/32
                    const uint2 v = *reinterpret_cast<const uint2*>(
                        rtile + pl * RROW + (((ocl >> 5) ^ rswz(pl, RROW / 16)) << 4) + ((ocl >> 4) & 1) * 8);
                    rw[0] = v.x; rw[1] = v.y;
                }
                if constexpr (F6) {   // fp32 sums of integers below 2^24: exact conversion
                    v16i ai;
#pragma unroll
                    for (int q = 0; q < 16; ++q) ai[q] = (int)accf[t][u][q];
                    epi_store16<true, RES ? 3 : 2>(p, ai, &cbias[ocl], mult, rw, ocb, pix, add, m_res);
                } else if constexpr (W4) {   // 16 * acc: back to acc, exactly
                    const v16i a = acc[t][u] >> 4;
                    epi_store16<false, RES ? 3 : 2, OUTK == 4, OUTK == 4 ? 1 : OUTK>(p, a, nullptr, mult, rw, ocb,
                                                                                  pix, add, m_res, irq32);
                } else {
                    epi_store16<false, RES ? (B4 ? 3 : 1) : 2, OUTK == 4, OUTK == 4 ? 1 : OUTK>(
                        p, acc[t][u], nullptr, mult, rw, ocb, pix, add, m_res, irq32);
                }
            }
        }
        init_acc();
        if (RES) {
            advance();
            if (!last_tile) sync();
        }
        if (!last_tile) {
            if constexpr (SP) read_sp(ring + cur_off, fx);
            else if constexpr (F6) read_f6(ring + cur_off, gx);
            else read_frags(ring + cur_off, foff0, fa0, fb0);
        }
    }
    // no DMA may still be writing this workgroup's LDS when it ends
    IQNN_WAIT_VM(0);
}

// ============================================================ fused 1x1 pair
// Two 1x1 convolutions over the same pixels, the second reading the first's output:
// y_a = requant(conv_a(x) + residual), the last conv of a bottleneck block (64 -> 256
// channels, Conv_Add / Conv_Add_Relu), and y_b = requant(conv_b(y_a)), the first conv
// of the next block (256 -> CC channels, Conv / Conv_Relu).  y_a is stored for the
// next block's residual and kept in LDS, 64 channels at a time, as conv_b's activation
// operand, so conv_b never reads it back from HBM.  Per tile of 128 pixels, stages of
// one ring:
//   X      the tile's x rows (128 x 64 bytes): all of conv_a's 256 output channels
//          (weights resident in LDS) into the accumulators;
//   R_j    residual channels 64j..64j+63 of the tile: their epilogue, the codes stored
//          to y_a and kept in LDS;
//   W_j    conv_b's weights for input channels 64j.. (CC rows x 64 bytes of its
//          tile-order copy): conv_b's K-step over the kept codes.
// With CC = 64 conv_b's 16 KB of weights stay in LDS instead (and conv_a's fragments
// in registers, 32 per lane, which keeps the LDS at two workgroups per CU), so the ring
// carries only the X and R stages -- all of them HBM reads -- and a plain barrier hands
// each block of codes to conv_b.  Every stage is two 1 KB DMA instructions per wave, so,
// as in the streaming kernel, "stage g has landed" is vmcnt <= (kPrNST - 2) * 2 with the
// stages issued kPrNST - 1 ahead.
constexpr int kPrCa = 64, kPrCb = 256, kPrBN = 128;   // conv_a C_in and C_out; pixels per tile
constexpr int kPrNST = 6;                             // ring slots
constexpr int kPrSlot = 8192;                         // bytes per ring slot
constexpr int kPrChunks = kPrCb / 64;                 // conv_a's channel blocks = conv_b's K-stages

// XS: the 8-bit activations (x and the kept codes) take the uint8 sign flip; false when
// both are signed codes (x_xor == 0 for both convs).
template <int CC, bool XS>
__global__ __launch_bounds__(256, 2) void qconv_pair(const ConvParams pa, const ConvParams pb, int32_t n_tiles) {
    constexpr int K_LOADS = 2, D = kPrNST - 1;
    constexpr int TB = CC / 64;   // conv_b: 32-channel blocks per wave (waves split CC in two)
    constexpr bool WRES = CC == 64;   // conv_b's weights resident, conv_a's in registers
    constexpr int STAGES = WRES ? 1 + kPrChunks : 1 + 2 * kPrChunks;   // ring stages per tile
    static_assert(CC == 64 || CC == 128, "conv_b's output channels");
    static_assert(kPrBN * 64 == 4 * K_LOADS * 1024 && CC * 64 <= kPrSlot, "a stage is two KB per wave");
    __shared__ __attribute__((aligned(1024))) uint8_t wa[WRES ? 16 : kPrCb * 64];
    __shared__ __attribute__((aligned(1024))) uint8_t wb[WRES ? kPrChunks * CC * 64 : 16];   // [K-stage][CC rows][64]
    __shared__ __attribute__((aligned(1024))) uint8_t ring[kPrNST * kPrSlot];
    __shared__ __attribute__((aligned(1024))) uint8_t codes[kPrBN * 64];
    __shared__ __attribute__((aligned(16))) int32_t biasa[kPrCb];
    __shared__ __attribute__((aligned(16))) float multa[kPrCb];
    __shared__ __attribute__((aligned(16))) int32_t biasb[CC];
    __shared__ __attribute__((aligned(16))) float multb[CC];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wo = wave & 1, wp = wave >> 1;   // channel half, pixel half of the tile
    const int G = gridDim.x;
    const int J = ((int)blockIdx.x < n_tiles) ? (n_tiles - (int)blockIdx.x + G - 1) / G : 0;
    if (J <= 0) return;
    auto tile_px0 = [&](int i) -> int64_t { return (int64_t)((int)blockIdx.x + i * G) * kPrBN; };

    biasa[tid] = pa.bias[tid];
    multa[tid] = pa.mult[tid];
    if (tid < CC) {
        biasb[tid] = pb.bias[tid];
        multb[tid] = pb.mult[tid];
    }
    __syncthreads();
    // conv_a's weights have one K-stage, so its tile-order copy is their 16 KB LDS image;
    // conv_b's (CC = 64: one row block) are four 4 KB blocks, one per K-stage, in order
    {
        const int8_t* wsrc = WRES ? pb.w_tiled : pa.w_tiled;
        const void* src[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) src[i] = wsrc + (wave * 4 + i) * 1024 + lane * 16;
        dma16_seq<4>(lds_addr(WRES ? wb : wa) + wave * 4096, src);
    }

    // ------------------------------------------------------------ issue side
    // X and R stages: rows are pixels, lane -> row 16i + lane/4 of the wave's 32, slot
    // lane%4 holding 16-byte segment slot ^ swz(row) (the fragment reads undo it)
    const uint32_t ring0 = lds_addr(ring);
    int is_i = 0, is_k = 0, is_slot = 0;
    int64_t rowpix[K_LOADS];
    int seg[K_LOADS];
    auto set_rows = [&](int i) {
#pragma unroll
        for (int ii = 0; ii < K_LOADS; ++ii) {
            const int row = (wave * K_LOADS + ii) * 16 + (lane >> 2);
            const int64_t pix = tile_px0(i) + row;
            rowpix[ii] = pix < pa.m ? pix : pa.m - 1;
            seg[ii] = ((lane & 3) ^ swz(row)) * 16;
        }
    };
    set_rows(0);
    auto issue = [&]() {
        const void* src[K_LOADS];
        if (is_k == 0) {   // x rows of the tile
#pragma unroll
            for (int ii = 0; ii < K_LOADS; ++ii) src[ii] = pa.x + rowpix[ii] * kPrCa + seg[ii];
        } else {
            const int j = WRES ? is_k - 1 : (is_k - 1) >> 1;
            if (WRES || (is_k & 1)) {   // residual channels 64j..
#pragma unroll
                for (int ii = 0; ii < K_LOADS; ++ii) src[ii] = pa.res + rowpix[ii] * kPrCb + 64 * j + seg[ii];
            } else {          // conv_b's weight rows for input channels 64j.., 1 KB pieces
#pragma unroll
                for (int ii = 0; ii < K_LOADS; ++ii) {
                    const int q = (wave * K_LOADS + ii) & (CC / 16 - 1);   // piece of the CC x 64 image
                    src[ii] = pb.w_tiled + ((int64_t)((q >> 2) * kPrChunks + j) * 4096) + (q & 3) * 1024 + lane * 16;
                }
            }
        }
        dma16_seq<K_LOADS>(ring0 + is_slot * kPrSlot + wave * K_LOADS * 1024, src);
        is_slot = is_slot + 1 == kPrNST ? 0 : is_slot + 1;
        // advance; past the last stage the cursor stays there (it is issued again into
        // the next slot, keeping every stage's DMA count)
        if (is_k + 1 < STAGES) {
            ++is_k;
        } else if (is_i + 1 < J) {
            ++is_i;
            is_k = 0;
            set_rows(is_i);
        }
    };
    // the LDS stores and reads of a stage stay on their side of its barrier (the DMA's
    // asm statements after it carry memory clobbers; this one holds the stores before)
    auto sync = [&]() {
        asm volatile("" ::: "memory");
        IQNN_WAIT_VM_LGKM0((D - 1) * K_LOADS);
        __builtin_amdgcn_s_barrier();
        issue();
    };

    // ------------------------------------------------------------ compute side
    const int frow = lane & 31;
    const int foff[2] = {frow * 64 + (((lane >> 5) + 0) ^ swz(frow)) * 16,
                         frow * 64 + (((lane >> 5) + 2) ^ swz(frow)) * 16};
    const int hl = (lane >> 5) * 16;   // the lane's 16 channels within a 32-channel block
    v16i acca[kPrChunks][2], accb[TB][2];
    // WRES: conv_a's A fragments, row 64j + 32 wo + frow of its tile-order copy (block j)
    v4i waf[WRES ? kPrChunks : 1][2];
    if constexpr (WRES) {
#pragma unroll
        for (int j = 0; j < kPrChunks; ++j)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                waf[j][kk] = *reinterpret_cast<const v4i*>(pa.w_tiled + j * 4096 + 32 * wo * 64 + foff[kk]);
    }

    for (int i = 0; i < D; ++i) issue();
    const float m_res = *pa.m_res;
    int slot = 0;   // ring slot of the stage being consumed
    auto next_slot = [&]() { slot = slot + 1 == kPrNST ? 0 : slot + 1; };
    for (int it = 0; it < J; ++it) {
        const int64_t px0 = tile_px0(it);
        sync();   // X: the tile's x rows
        {
            const uint8_t* xt = ring + slot * kPrSlot;
#pragma unroll
            for (int j = 0; j < kPrChunks; ++j) {
                const int ca = 64 * j + 32 * wo + hl;
                v16i b;
#pragma unroll
                for (int q = 0; q < 16; ++q) b[q] = biasa[ca + q];
                acca[j][0] = b;
                acca[j][1] = b;
            }
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                v4i fb[2];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    fb[u] = *reinterpret_cast<const v4i*>(xt + (64 * wp + 32 * u) * 64 + foff[kk]);
                    if constexpr (XS) { fb[u][0] ^= pa.x_xor; fb[u][1] ^= pa.x_xor; fb[u][2] ^= pa.x_xor; fb[u][3] ^= pa.x_xor; }
                }
#pragma unroll
                for (int j = 0; j < kPrChunks; ++j) {
                    const v4i fa = WRES ? waf[j][kk] : *reinterpret_cast<const v4i*>(wa + (64 * j + 32 * wo) * 64 + foff[kk]);
#pragma unroll
                    for (int u = 0; u < 2; ++u)
                        acca[j][u] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa, fb[u], acca[j][u], 0, 0, 0);
                }
            }
        }
        next_slot();
#pragma unroll
        for (int t = 0; t < TB; ++t) {
            const int ob = wo * (CC / 2) + 32 * t + hl;
            v16i b;
#pragma unroll
            for (int q = 0; q < 16; ++q) b[q] = biasb[ob + q];
            accb[t][0] = b;
            accb[t][1] = b;
        }
#pragma unroll
        for (int j = 0; j < kPrChunks; ++j) {
            sync();   // R_j: the residual channels
            {
                const uint8_t* rt = ring + slot * kPrSlot;
                const int ocl = 32 * wo + hl;   // channel within the 64-channel block
                float mult[16];
#pragma unroll
                for (int q = 0; q < 16; ++q) mult[q] = multa[64 * j + ocl + q];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int pl = 64 * wp + 32 * u + frow;
                    const int64_t pix = px0 + pl;
                    if (pix < pa.m) {
                        const uint4 rv = *reinterpret_cast<const uint4*>(rt + pl * 64 + (((ocl >> 4) ^ swz(pl)) << 4));
                        uint32_t rw[4] = {rv.x, rv.y, rv.z, rv.w};
                        uint4 pk;
                        epi_store16<false, 1, false, 1>(pa, acca[j][u], nullptr, mult, rw, 64 * j + ocl, pix, true,
                                                        m_res, false, &pk);
                        *reinterpret_cast<uint4*>(codes + pl * 64 + (((ocl >> 4) ^ swz(pl)) << 4)) = pk;
                    }
                }
            }
            next_slot();
            if constexpr (WRES) {   // the codes are complete: LDS stores done, then the barrier
                asm volatile("" ::: "memory");
                __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt left at their maximum
                __builtin_amdgcn_s_barrier();
                asm volatile("" ::: "memory");
            } else {
                sync();   // W_j: conv_b's weights for these 64 input channels; the codes are complete
            }
            {
                const uint8_t* wt = WRES ? wb + j * CC * 64 : ring + slot * kPrSlot;
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    v4i fb[2];
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        fb[u] = *reinterpret_cast<const v4i*>(codes + (64 * wp + 32 * u) * 64 + foff[kk]);
                        if constexpr (XS) { fb[u][0] ^= pb.x_xor; fb[u][1] ^= pb.x_xor; fb[u][2] ^= pb.x_xor; fb[u][3] ^= pb.x_xor; }
                    }
#pragma unroll
                    for (int t = 0; t < TB; ++t) {
                        const v4i fa = *reinterpret_cast<const v4i*>(wt + (wo * (CC / 2) + 32 * t) * 64 + foff[kk]);
#pragma unroll
                        for (int u = 0; u < 2; ++u)
                            accb[t][u] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa, fb[u], accb[t][u], 0, 0, 0);
                    }
                }
            }
            if constexpr (!WRES) next_slot();
        }
        // conv_b's epilogue
#pragma unroll
        for (int t = 0; t < TB; ++t) {
            const int ob = wo * (CC / 2) + 32 * t + hl;
            float mult[16];
#pragma unroll
            for (int q = 0; q < 16; ++q) mult[q] = multb[ob + q];
            uint32_t rw[4] = {0, 0, 0, 0};
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int64_t pix = px0 + 64 * wp + 32 * u + frow;
                if (pix < pb.m) epi_store16<false, 2, false, 1>(pb, accb[t][u], nullptr, mult, rw, ob, pix, false, 0.0f);
            }
        }
    }
    // no DMA may still be writing this workgroup's LDS when it ends
    IQNN_WAIT_VM(0);
}

// Persistent schedule of the streaming kernel over the 8 XCDs (workgroup ids are dealt
// round-robin, so workgroup i runs on XCD i % 8).  The channel tiles are split into
// xo_groups groups (1, 2, 4 or 8, dividing the tile count) and the pixel tiles into
// 8 / xo_groups shares; XCD x takes group x % xo_groups and share x / xo_groups.  Its
// workgroups, about occ per CU (32 CUs per XCD) and a multiple of its channel tiles,
// each keep one channel tile and walk a strided run of the share's pixel tiles.
// xo_groups > 1 keeps an XCD's weights (its channel groups' rows) resident in its 4 MB
// L2 when all of a layer's weights are too large for that; the rule takes the
// smallest split that brings them to at most kXcdWeightBytes.
constexpr int64_t kXcdWeightBytes = 2 << 20;
void stream_schedule(ConvParams& q, int occ) {
    const int n_oc_all = q.n_oc_tiles;
    int xo = 1;
    const int forced = q.xcd_force;
    if (forced > 0) {
        xo = forced;
    } else {
        const int64_t w_bytes = (int64_t)q.c_out * q.kp * (q.w_idx ? 5 : 8) / 8;
        while (xo < 8 && w_bytes / xo > kXcdWeightBytes && n_oc_all % (2 * xo) == 0) xo *= 2;
    }
    while (xo > 1 && n_oc_all % xo != 0) xo /= 2;
    q.xo_groups = xo;
    const int n_oc = n_oc_all / xo;
    const int shares = 8 / xo;
    q.px_chunk = (int32_t)((q.n_px_tiles + shares - 1) / shares);
    int per = n_oc * std::max(1, occ * 32 / n_oc);
    per = (int)std::min<int64_t>(per, (int64_t)q.px_chunk * n_oc);
    q.gx = per;
}

// 4-bit activations (packed rows streamed to LDS): the 64x128 and 128x128 blocks; F6:
// INT4 weights as BF6 on the FP6 MFMA (ConvParams::f6 set by the host).
template <class C, bool F6, bool S4 = false, bool W4 = false>
hipError_t launch_stream_b4_k(const ConvParams& q, dim3 g, dim3 b, bool is_1x1, hipStream_t stream) {
    const bool add = q.epi == E_ADD || q.epi == E_ADD_RELU;
    if (is_1x1 && add) hipLaunchKernelGGL((qconv_stream<C, true, true, false, true, false, false, F6, 0, S4, W4>), g, b, 0, stream, q);
    else if (is_1x1) hipLaunchKernelGGL((qconv_stream<C, true, false, false, true, false, false, F6, 0, S4, W4>), g, b, 0, stream, q);
    else if (add) hipLaunchKernelGGL((qconv_stream<C, false, true, false, true, false, false, F6, 0, S4, W4>), g, b, 0, stream, q);
    else hipLaunchKernelGGL((qconv_stream<C, false, false, false, true, false, false, F6, 0, S4, W4>), g, b, 0, stream, q);
    return hipGetLastError();
}

// F6: the FP6 path; otherwise the activations' signedness and the packed INT4 weights
// (ConvParams::w4, set by the host) select the compiled variant.
template <class C, bool F6>
hipError_t launch_stream_b4(const ConvParams& p, bool is_1x1, hipStream_t stream) {
    ConvParams q = p;
    q.n_oc_tiles = (p.c_out + C::BM - 1) / C::BM;
    const int64_t n_px = (p.m + C::BN - 1) / C::BN;
    if (n_px <= 0) return hipSuccess;
    if (p.m >= ((int64_t)1 << 31) || (!is_1x1 && p.kh * p.kw > 64)) return hipErrorInvalidValue;
    q.n_px_tiles = (int32_t)n_px;
    stream_schedule(q, C::OCC);
    dim3 g((unsigned)(8 * q.gx)), b(256);
    if constexpr (F6) {
        return launch_stream_b4_k<C, true>(q, g, b, is_1x1, stream);
    } else {
        if (p.w4) {
            if constexpr (C::BM % 128 == 0) {
                return p.x_signed4 ? launch_stream_b4_k<C, false, true, true>(q, g, b, is_1x1, stream)
                                   : launch_stream_b4_k<C, false, false, true>(q, g, b, is_1x1, stream);
            }
            return hipErrorInvalidValue;
        }
        return p.x_signed4 ? launch_stream_b4_k<C, false, true>(q, g, b, is_1x1, stream)
                           : launch_stream_b4_k<C, false, false>(q, g, b, is_1x1, stream);
    }
}

// A block reads weight rows [oc0, oc0 + BM) of the packed layer, whose channels are
// padded to a multiple of kOcPad: blocks wider than that need the padded count to be a
// multiple of their width, or the last block would read past the packed buffer.
bool block_fits_packed(int32_t c_out, int bm) {
    const int64_t ocp = ((int64_t)c_out + kOcPad - 1) / kOcPad * kOcPad;
    return bm <= kOcPad ? kOcPad % bm == 0 : ocp % bm == 0;
}

// The block configurations compiled with the integer-only requantization (specialized
// beside the tile table below).
template <class C> constexpr bool kIrqTile = false;

template <class C>
hipError_t launch_stream(const ConvParams& p, bool is_1x1, bool res_prefetch, bool c4, hipStream_t stream,
                         bool zw = false) {
    if (!block_fits_packed(p.c_out, C::BM)) return hipErrorInvalidValue;
    ConvParams q = p;
    q.n_oc_tiles = (p.c_out + C::BM - 1) / C::BM;
    const int64_t n_px = (p.m + C::BN - 1) / C::BN;
    if (n_px <= 0) return hipSuccess;
    if (p.m >= ((int64_t)1 << 31) || (!is_1x1 && !c4 && p.kh * p.kw > 64)) return hipErrorInvalidValue;
    q.n_px_tiles = (int32_t)n_px;
    stream_schedule(q, C::OCC);
    dim3 g((unsigned)(8 * q.gx)), b(64 * C::NW);
    if (zw) {   // asymmetric weights: the 64x256 and 128x128 configurations only
        if constexpr (C::OCC < 3 && ((C::BN == 256 && C::BM == 64 && C::NST == 3) ||
                                     (C::BN == 128 && C::BM == 128 && C::NST == 4))) {
            const bool add = p.epi == E_ADD || p.epi == E_ADD_RELU;
            if (c4 || (add && !res_prefetch)) return hipErrorInvalidValue;
            if (is_1x1 && add) hipLaunchKernelGGL((qconv_stream<C, true, true, false, false, true>), g, b, 0, stream, q);
            else if (is_1x1) hipLaunchKernelGGL((qconv_stream<C, true, false, false, false, true>), g, b, 0, stream, q);
            else if (add) hipLaunchKernelGGL((qconv_stream<C, false, true, false, false, true>), g, b, 0, stream, q);
            else hipLaunchKernelGGL((qconv_stream<C, false, false, false, false, true>), g, b, 0, stream, q);
            return hipGetLastError();
        }
        return hipErrorInvalidValue;
    }
    if constexpr (C::NW == 4 && (C::NST - 1) * (C::BM / 64 + C::BN / 16) <= 60 && C::OCC < 3) {
        if (c4) {
            hipLaunchKernelGGL((qconv_stream<C, false, false, true>), g, b, 0, stream, q);
            return hipGetLastError();
        }
    } else if (c4) {
        return hipErrorInvalidValue;
    }
    // the residual rides in the stream when a tile of it fits one stage
    constexpr bool kResStage = C::BM * C::BN <= (C::BM + C::BN) * kPipeBK && C::OCC < 3;
    const bool add = p.epi == E_ADD || p.epi == E_ADD_RELU;
    if (add && !(kResStage && res_prefetch)) return hipErrorInvalidValue;
    // 8-bit codes stored 16 channels at a time: the epilogue compiled for that output
    const bool out8 = p.epi != E_RAW && (p.y_type == T_INT8 || p.y_type == T_UINT8) && p.vec_store;
    if (p.int_rq) {   // integer-only requantization: Conv / Conv_Relu to 8-bit codes
        if (!kIrqTile<C> || add || !out8 || c4) return hipErrorInvalidValue;
        if constexpr (kIrqTile<C>) {
            if (is_1x1)
                hipLaunchKernelGGL((qconv_stream<C, true, false, false, false, false, false, false, 4>), g, b, 0, stream, q);
            else
                hipLaunchKernelGGL((qconv_stream<C, false, false, false, false, false, false, false, 4>), g, b, 0, stream, q);
            return hipGetLastError();
        }
    }
    // KxK layers without a residual whose tiles have more than D + 1 stages: the split
    // stage loop (the issue side's tile switch between two loops)
    const bool split = !is_1x1 && !c4 && !add && p.kh * p.kw <= 32 && p.kp / kPipeBK > C::NST;
    // ring rounds: signed codes on rings of at most 4 slots (unrolled with the sign flip,
    // or over 6 slots, the compiler spills)
    const bool rounds = split && (p.kp / kPipeBK) % C::NST == 0 && C::NST <= 4;
    // signed 8-bit activations on the automatic choice's configurations: no sign flip
    if constexpr (kIrqTile<C>) {
        if (out8 && p.x_xor == 0u && !(add && !kResStage)) {
            if constexpr (kResStage) {
                if (add && is_1x1)
                    hipLaunchKernelGGL((qconv_stream<C, true, true, false, false, false, false, false, 1, false, false, false>),
                                       g, b, 0, stream, q);
                else if (add)
                    hipLaunchKernelGGL((qconv_stream<C, false, true, false, false, false, false, false, 1, false, false, false>),
                                       g, b, 0, stream, q);
            }
            if (!add && is_1x1)
                hipLaunchKernelGGL((qconv_stream<C, true, false, false, false, false, false, false, 1, false, false, false>),
                                   g, b, 0, stream, q);
            else if (!add && rounds)
                hipLaunchKernelGGL((qconv_stream<C, false, false, false, false, false, false, false, 1, false, false, false,
                                                 C::NST <= 4 ? 2 : 1>), g, b, 0, stream, q);
            else if (!add && split)
                hipLaunchKernelGGL((qconv_stream<C, false, false, false, false, false, false, false, 1, false, false, false, 1>),
                                   g, b, 0, stream, q);
            else if (!add)
                hipLaunchKernelGGL((qconv_stream<C, false, false, false, false, false, false, false, 1, false, false, false>),
                                   g, b, 0, stream, q);
            return hipGetLastError();
        }
    }
    if constexpr (kResStage) {
        if (res_prefetch) {
            if (is_1x1 && out8)
                hipLaunchKernelGGL((qconv_stream<C, true, true, false, false, false, false, false, 1>), g, b, 0, stream, q);
            else if (is_1x1)
                hipLaunchKernelGGL((qconv_stream<C, true, true, false>), g, b, 0, stream, q);
            else if (out8)
                hipLaunchKernelGGL((qconv_stream<C, false, true, false, false, false, false, false, 1>), g, b, 0, stream, q);
            else
                hipLaunchKernelGGL((qconv_stream<C, false, true, false>), g, b, 0, stream, q);
            return hipGetLastError();
        }
    }
    if (is_1x1 && out8)
        hipLaunchKernelGGL((qconv_stream<C, true, false, false, false, false, false, false, 1>), g, b, 0, stream, q);
    else if (is_1x1)
        hipLaunchKernelGGL((qconv_stream<C, true, false, false>), g, b, 0, stream, q);
    else if (out8 && split && kIrqTile<C>)
        hipLaunchKernelGGL((qconv_stream<C, false, false, false, false, false, false, false, 1, false, false, true,
                                         kIrqTile<C> ? 1 : 0>), g, b, 0, stream, q);
    else if (out8)
        hipLaunchKernelGGL((qconv_stream<C, false, false, false, false, false, false, false, 1>), g, b, 0, stream, q);
    else
        hipLaunchKernelGGL((qconv_stream<C, false, false, false>), g, b, 0, stream, q);
    return hipGetLastError();
}

// Block configuration of the 2:4 kernel: a stage is 40 bytes per weight row (kept
// codes + positions) and 64 per pixel row.
template <int BM_, int BN_, int WM_, int NST_>
struct StreamCfg2of4 {
    static constexpr int NW = 4;
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = 4 / WM_, NST = NST_;
    static constexpr int WOC = BM / WM, WPX = BN / WN;
    static constexpr int TM = WOC / 32, TN = WPX / 32;
    static constexpr int STAGE = BM * 40 + BN * kPipeBK;
    static constexpr int LDS = NST * STAGE + 8 * BM;
    static constexpr int OCC = 160 * 1024 / LDS >= 2 ? 2 : 1;
};

// 2:4-sparse weights: 128x128 blocks, two per CU (199-236 VGPRs), the schedule of the
// dense streaming kernel.  Without a residual the 13 KB stages allow a ring of 6 (five
// stages in flight); the residual stage needs 16 KB slots, so a ring of 4.
template <class C>
hipError_t launch_stream_2of4_cfg(const ConvParams& p, bool is_1x1, hipStream_t stream) {
    ConvParams q = p;
    q.n_oc_tiles = (p.c_out + C::BM - 1) / C::BM;
    const int64_t n_px = (p.m + C::BN - 1) / C::BN;
    if (n_px <= 0) return hipSuccess;
    if (p.m >= ((int64_t)1 << 31) || (!is_1x1 && p.kh * p.kw > 64)) return hipErrorInvalidValue;
    q.n_px_tiles = (int32_t)n_px;
    stream_schedule(q, C::OCC);
    dim3 g((unsigned)(8 * q.gx)), b(256);
    const bool add = p.epi == E_ADD || p.epi == E_ADD_RELU;
    if constexpr (C::NST * C::BN * C::BM + 8 * C::BM <= 80 * 1024) {   // residual slots fit two per CU
        if (is_1x1 && add) hipLaunchKernelGGL((qconv_stream<C, true, true, false, false, false, true>), g, b, 0, stream, q);
        else if (add) hipLaunchKernelGGL((qconv_stream<C, false, true, false, false, false, true>), g, b, 0, stream, q);
    } else if (add) {
        return hipErrorInvalidValue;
    }
    if (!add) {
        if (is_1x1) hipLaunchKernelGGL((qconv_stream<C, true, false, false, false, false, true>), g, b, 0, stream, q);
        else hipLaunchKernelGGL((qconv_stream<C, false, false, false, false, false, true>), g, b, 0, stream, q);
    }
    return hipGetLastError();
}

hipError_t launch_stream_2of4(const ConvParams& p, bool is_1x1, hipStream_t stream) {
    const bool add = p.epi == E_ADD || p.epi == E_ADD_RELU;
    if (add) return launch_stream_2of4_cfg<StreamCfg2of4<128, 128, 2, 4>>(p, is_1x1, stream);
    return launch_stream_2of4_cfg<StreamCfg2of4<128, 128, 2, 6>>(p, is_1x1, stream);
}

// ============================================================ stem kernel
//
// qconv_stem: the image stem (4-channel input laid out by iqnn_quantize_pad, filter
// rows widened to 8 taps, stride 2, C_out <= 64) as a direct convolution.  A tile is
// 128 consecutive output pixels of one image; the input rows they need (at most
// max_rows) are one contiguous byte range, copied into LDS with 16-byte DMA while
// the previous tile computes (two buffers).  Each wave holds the A fragments of all
// 64 channels and every filter row in registers for its whole life, and builds the
// B fragment of filter row ky straight from the slab: pixel (oy, ox), taps
// 4h..4h+3 of row ky are 16 consecutive bytes at slab row 2(oy-oy0)+ky, column 2ox+4h.
// One 32-byte k-step per filter row: K = 7 x 8 x 4 = 224, no per-tap gather.
constexpr int kStemBN = 128;
constexpr int kStemBuf = 12288;   // LDS bytes per slab buffer (12 DMA instructions of 1 KB)
constexpr int kStemKH = 8;        // filter rows held in registers

__global__ __launch_bounds__(256, 3) void qconv_stem(const ConvParams p, int32_t n_tiles, int64_t in_bytes) {
    __shared__ __attribute__((aligned(1024))) uint8_t slab[2][kStemBuf];
    __shared__ __attribute__((aligned(16))) int32_t cbias[64];
    __shared__ __attribute__((aligned(16))) float cmult[64];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    if ((int)blockIdx.x >= n_tiles) return;
    if (tid < 64) {
        cbias[tid] = p.bias[tid];
        cmult[tid] = p.mult[tid];
    }
    // A fragments: packed rows 32t + lane%32, K bytes 32 ky + 16 (lane/32)
    v4i wa[2][kStemKH];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int ky = 0; ky < kStemKH; ++ky)
            wa[t][ky] = ky < p.kh ? *reinterpret_cast<const v4i*>(p.w + (int64_t)(32 * t + (lane & 31)) * p.kp +
                                                                  32 * ky + 16 * (lane >> 5))
                                  : v4i{0, 0, 0, 0};
    __syncthreads();

    const uint32_t ohw = (uint32_t)(p.oh * p.ow);
    const int64_t row_bytes = (int64_t)p.w_in * 4;
    auto slab_start = [&](int tile, int64_t& start, uint32_t& oy0) {
        const uint32_t P0 = (uint32_t)tile * kStemBN;
        const uint32_t n = P0 / ohw, pix0 = P0 - n * ohw;
        oy0 = pix0 / (uint32_t)p.ow;
        start = ((int64_t)n * p.h + 2 * (int64_t)oy0) * row_bytes;   // 8-byte aligned (W even)
    };
    auto issue = [&](int tile, int buf) {
        int64_t start;
        uint32_t oy0;
        slab_start(tile, start, oy0);
        const int64_t base = start & ~(int64_t)15;
        for (int j = wave; j < kStemBuf / 1024; j += 4) {
            const int64_t off = base + j * 1024 + lane * 16;
            const void* src = off + 16 <= in_bytes ? (const void*)(p.x + off) : (const void*)p.x;
            dma16_run<1>(lds_addr(&slab[buf][0]) + j * 1024, &src);
        }
    };

    v16i acc[2];
    const int frow = lane & 31;
    const uint32_t bxor = p.x_xor;
    int buf = 0;
    issue(blockIdx.x, 0);
    for (int tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
        // this tile's slab has landed (and every wave is done with the other buffer)
        IQNN_WAIT_VM_LGKM0(0);
        __builtin_amdgcn_s_barrier();
        const int next = tile + (int)gridDim.x;
        if (next < n_tiles) issue(next, buf ^ 1);

        int64_t start;
        uint32_t oy0;
        slab_start(tile, start, oy0);
        const uint32_t shift = (uint32_t)(start & 15);
        const uint32_t P0 = (uint32_t)tile * kStemBN;
        const uint32_t pl = wave * 32 + frow;               // pixel inside the tile
        const uint32_t pix = (P0 % ohw) + pl;
        const uint32_t oy = pix / (uint32_t)p.ow, ox = pix - oy * (uint32_t)p.ow;
        const uint32_t b0 = shift + (uint32_t)((2 * (oy - oy0)) * row_bytes) + ox * 8 + 16 * (lane >> 5);
        const uint2* sv = reinterpret_cast<const uint2*>(&slab[buf][0]);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int ocl = t * 32 + (lane >> 5) * 16;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int4 bv = *reinterpret_cast<const int4*>(&cbias[ocl + 4 * q]);
                acc[t][4 * q] = bv.x; acc[t][4 * q + 1] = bv.y; acc[t][4 * q + 2] = bv.z; acc[t][4 * q + 3] = bv.w;
            }
        }
#pragma unroll
        for (int ky = 0; ky < kStemKH; ++ky) {
            if (ky < p.kh) {
                const uint32_t a = (b0 + ky * (uint32_t)row_bytes) >> 3;   // 8-byte units
                const uint2 lo = sv[a], hi = sv[a + 1];
                v4i fb = {(int)(lo.x ^ bxor), (int)(lo.y ^ bxor), (int)(hi.x ^ bxor), (int)(hi.y ^ bxor)};
                acc[0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(wa[0][ky], fb, acc[0], 0, 0, 0);
                acc[1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(wa[1][ky], fb, acc[1], 0, 0, 0);
            }
        }
        const int64_t opix = (int64_t)P0 + pl;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int ocb = t * 32 + (lane >> 5) * 16;
            if (ocb >= p.c_out) continue;
            float mult[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 mv = *reinterpret_cast<const float4*>(&cmult[ocb + 4 * q]);
                mult[4 * q] = mv.x; mult[4 * q + 1] = mv.y; mult[4 * q + 2] = mv.z; mult[4 * q + 3] = mv.w;
            }
            uint32_t rw[4] = {0, 0, 0, 0};
            epi_store16<false, 2>(p, acc[t], nullptr, mult, rw, ocb, opix, false, 0.0f);
        }
        buf ^= 1;
    }
    // no DMA may still be writing this workgroup's LDS when it ends
    IQNN_WAIT_VM(0);
}

// The stem kernel's conditions (see qconv_stem): 4-channel gather with 8-tap rows,
// stride 2, at most kStemKH filter rows, C_out <= 64 in 16-channel groups, whole
// 128-pixel tiles per image, an even input width (8-byte aligned slab reads), a
// slab that fits one buffer, no residual, and an input of whole 16-byte units: the
// slab DMA moves 16 bytes per lane from a 16-byte aligned start, and a unit that ran
// past the end of the input (N*H*W*4 = 8 mod 16) would still hold needed bytes.
bool stem_ok(const ConvParams& p) {
    if (p.kw != 8 || p.sh != 2 || p.sw != 2 || p.kh > kStemKH || p.c_out > 64 || !p.vec_store) return false;
    if (p.epi == E_ADD || p.epi == E_ADD_RELU) return false;
    const int64_t ohw = (int64_t)p.oh * p.ow;
    if (ohw % kStemBN != 0 || p.w_in % 2 != 0 || p.m >= ((int64_t)1 << 31)) return false;
    if ((p.m / ohw) * p.h * (int64_t)p.w_in * 4 % 16 != 0) return false;
    const int64_t out_rows = (kStemBN - 1 + p.ow - 1) / p.ow + 1;   // output rows one tile can touch
    const int64_t max_rows = 2 * (out_rows - 1) + p.kh;
    return max_rows * p.w_in * 4 + 16 <= kStemBuf;
}

hipError_t launch_stem(const ConvParams& p, hipStream_t stream) {
    const int64_t n_tiles = p.m / kStemBN;
    if (n_tiles <= 0) return hipSuccess;
    const int64_t in_bytes = p.m / ((int64_t)p.oh * p.ow) * p.h * (int64_t)p.w_in * 4;
    const int64_t grid = std::min<int64_t>(n_tiles, 256 * 3);
    hipLaunchKernelGGL(qconv_stem, dim3((unsigned)grid), dim3(256), 0, stream, p, (int32_t)n_tiles, in_bytes);
    return hipGetLastError();
}

// ============================================================ stem + max pooling
//
// qconv_stem_pool: the stem convolution of qconv_stem followed by max pooling 3x3,
// stride 2, padding 1, without writing the convolution's output.  The requantizing
// epilogue y(a) = clip(rne(float(a) * M[c]) + Z_out) is a non-decreasing function of
// the int32 accumulator a of channel c (M[c] > 0, and the conversion, the product, the
// rounding and the clip each preserve order), so the max of y over a pooling window is
// y of the max of a over it: the kernel pools the accumulators and requantizes only
// the pooled values -- a quarter of the stem's outputs -- and the bytes equal those of
// pooling the stored stem codes (max pooling is passive on codes, "Quantization" blog,
// 量化激活函数).
// Wave g of a workgroup owns pooled columns 31g .. 31g+30 of one image; the workgroup
// owns a band of pooled rows.  For every stem row, lane l (j = l % 32, pooled column
// c = 31g + j) computes two MFMA blocks: stem column 2c-1 (block 0) and 2c (block 1),
// each for all 64 channels.  The window of pooled column c is stem columns 2c-1, 2c,
// 2c+1, and 2c+1 is block 0 of lane l+1, shuffled over; lanes 31 and 63 only feed
// their left neighbour.  Out-of-image window columns are replaced by an in-image
// column of the same window (column -1 by column 0), which leaves the max unchanged.
// The window's stem rows are 2r-1, 2r, 2r+1; row 2r+1 stays in registers as the next
// pooled row's first row.  The input rows of a stem row pair are one contiguous byte
// range, copied into LDS with 16-byte DMA kSpAhead pairs ahead through kSpSlabs slab
// buffers; every wave issues exactly kSpCpw(NW) DMA instructions per slab (chunks past
// the end repeat the last chunk: the same bytes to the same place), so "slab r landed"
// is vmcnt <= (kSpAhead-1)*kSpCpw while the later slabs are in flight.
constexpr int kSpBuf = 9216;       // LDS bytes per slab buffer
constexpr int kSpAhead = 3;        // row pairs in flight
constexpr int kSpSlabs = kSpAhead + 1;
constexpr int kSpColsPerWave = 31; // pooled columns per wave
constexpr int kSpMaxWaves = 4;     // pooled width limit 124
constexpr int kSpCpw(int nw) { return (kSpBuf / 1024 + nw - 1) / nw; }

struct StemPoolArgs {
    uint8_t* yp;                   // pooled output [N][PH][PW][64]
    int32_t ph, pw;                // pooled height, width
    int32_t band, n_bands;         // pooled rows per workgroup, workgroups per image
    int64_t in_bytes;              // size of the input tensor (whole 16-byte units)
};

// KH: filter rows (0: p.kh at run time); XX: the input bytes take the XOR with p.x_xor
// (unsigned codes), without it they are used as they are; FIX: the odd part of Z_out
// added to each rounded code (0 or 1 = p.out_fix, -1: p.out_fix read at run time), so
// that no branch splits the loop body.
template <int NW, int KH, bool XX, int FIX>
__global__ __launch_bounds__(64 * NW, NW == 1 ? 1 : 2) void qconv_stem_pool(const ConvParams p, const StemPoolArgs a) {
    constexpr int CPW = kSpCpw(NW);
    constexpr int KR = KH > 0 ? KH : kStemKH;   // filter rows held in registers
    static_assert((kSpAhead - 1) * CPW <= 60, "DMA in flight must fit the 6-bit vmcnt");
    static_assert(KR <= kStemKH, "filter rows");
    __shared__ __attribute__((aligned(1024))) uint8_t slab[kSpSlabs][kSpBuf];
    __shared__ __attribute__((aligned(16))) int32_t cbias[64];
    __shared__ __attribute__((aligned(16))) float cmult[64];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kh = KH > 0 ? KH : p.kh;
    const int n = (int)blockIdx.x / a.n_bands;
    const int r0 = ((int)blockIdx.x - n * a.n_bands) * a.band;
    const int r1 = min(a.ph, r0 + a.band);
    if (r0 >= r1) return;
    if (tid < 64) {
        cbias[tid] = p.bias[tid];
        cmult[tid] = p.mult[tid];
    }
    v4i wa[2][KR];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int ky = 0; ky < KR; ++ky)
            wa[t][ky] = ky < kh ? *reinterpret_cast<const v4i*>(p.w + (int64_t)(32 * t + (lane & 31)) * p.kp +
                                                               32 * ky + 16 * (lane >> 5))
                                : v4i{0, 0, 0, 0};
    __syncthreads();

    const int ow = p.ow;
    const int64_t row_bytes = (int64_t)p.w_in * 4;
    // copy input rows [2*sr0, 2*sr0 + nrows) of image n into slab buffer `buf`: chunk j
    // is 1 KB from the wave-uniform address p.x + base + 1024 j, each lane 16 bytes at
    // its own offset (the input is below 2 GB, so 32-bit offsets reach all of it)
    const uint32_t in_bytes = (uint32_t)a.in_bytes;
    auto issue = [&](int sr0, int nrows, int buf) {
        const uint32_t start = (uint32_t)(((int64_t)n * p.h + 2 * (int64_t)sr0) * row_bytes);
        const uint32_t base = start & ~15u;
        const int chunks = (int)((start - base + (uint32_t)(nrows * row_bytes) + 1023) >> 10);   // <= kSpBuf / 1024
#pragma unroll
        for (int i = 0; i < CPW; ++i) {
            const int j = min(wave + i * NW, chunks - 1);
            const uint32_t c0 = base + (uint32_t)j * 1024;
            uint32_t voff = c0 + (uint32_t)lane * 16;
            // a unit past the end of the input holds no needed byte (the input is whole
            // 16-byte units): it reads the first unit instead
            if (c0 + 1024 > in_bytes) voff = voff + 16 <= in_bytes ? voff : 0u;
            dma16_sbase(lds_addr(&slab[buf][0]) + j * 1024, p.x, voff);
        }
    };
    // This lane's pooled column pc and its two stem columns u (block 0) and u + 1
    // (block 1), u = 2pc - 1 clamped into [0, OW-1].  Column u + 1 sits 8 bytes after
    // column u, so a filter row of both blocks is three 8-byte units.  Clamping changes
    // nothing that is used: at pc = 0 the blocks are columns 0 and 1 (the window's
    // in-image columns are 0 and 1); a clamped u = OW-1 only occurs on lanes past the
    // pooled width, whose block 1 (the partial column OW, read inside the slab) is never
    // used, while their block 0 -- used by the lane to their left -- is unclamped.
    const int jl = lane & 31;
    const int pc = kSpColsPerWave * wave + jl;
    const uint32_t u = (uint32_t)min(max(2 * pc - 1, 0), ow - 1);
    const uint32_t bxor = XX ? p.x_xor : 0u;
    // accumulators of stem row sr (slab buffer `buf` starts at input row 2*sr0): blocks
    // b (stem columns u, u + 1) x channel halves t, the first MFMA adding to the bias
    auto stem_row = [&](int sr, int sr0, int buf, v16i (&acc)[2][2]) {
        const int64_t start = ((int64_t)n * p.h + 2 * (int64_t)sr0) * row_bytes;
        const uint32_t rb = (uint32_t)(start & 15) + (uint32_t)(2 * (sr - sr0) * row_bytes) + 16 * (lane >> 5) + 8 * u;
        const uint2* sv = reinterpret_cast<const uint2*>(&slab[buf][0]);
#pragma unroll
        for (int ky = 0; ky < KR; ++ky) {
            if (ky == 0 || KH > 0 || ky < kh) {   // kh >= 1
                const uint32_t ad = (rb + ky * (uint32_t)row_bytes) >> 3;
                const uint2 q0 = sv[ad], q1 = sv[ad + 1], q2 = sv[ad + 2];
                v4i f0, f1;
                if constexpr (XX) {
                    const uint32_t m0 = q1.x ^ bxor, m1 = q1.y ^ bxor;
                    f0 = v4i{(int)(q0.x ^ bxor), (int)(q0.y ^ bxor), (int)m0, (int)m1};
                    f1 = v4i{(int)m0, (int)m1, (int)(q2.x ^ bxor), (int)(q2.y ^ bxor)};
                } else {
                    f0 = v4i{(int)q0.x, (int)q0.y, (int)q1.x, (int)q1.y};
                    f1 = v4i{(int)q1.x, (int)q1.y, (int)q2.x, (int)q2.y};
                }
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    if (ky == 0) {   // both blocks start from the bias of channels ocl .. ocl+15
                        const int ocl = t * 32 + (lane >> 5) * 16;
                        v16i bias;
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int4 bv = *reinterpret_cast<const int4*>(&cbias[ocl + 4 * q]);
                            bias[4 * q] = bv.x; bias[4 * q + 1] = bv.y; bias[4 * q + 2] = bv.z; bias[4 * q + 3] = bv.w;
                        }
                        acc[0][t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(wa[t][ky], f0, bias, 0, 0, 0);
                        acc[1][t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(wa[t][ky], f1, bias, 0, 0, 0);
                    } else {
                        acc[0][t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(wa[t][ky], f0, acc[0][t], 0, 0, 0);
                        acc[1][t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(wa[t][ky], f1, acc[1][t], 0, 0, 0);
                    }
                }
            }
        }
    };

    const int kr = kh + 2;   // input rows of a stem row pair
    const bool store = jl < kSpColsPerWave && pc < a.pw;
    // requantized bytes of pooled maxima h (channel halves t, 16 channels each)
    auto requant = [&](const int32_t (&h)[2][16], uint4 (&pk)[2]) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int ocb = t * 32 + (lane >> 5) * 16;
            uint32_t bb[16];
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const float v = (float)h[t][q] * cmult[ocb + q];
                bb[q] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_fmed3f(v, p.t_lo, p.t_hi) + p.out_magic) +
                        (FIX < 0 ? p.out_fix : (uint32_t)FIX);
            }
            pk[t] = pack_bytes16(p, bb);
        }
    };
    auto put = [&](int r, const uint4 (&pk)[2]) {
        uint8_t* dst = a.yp + (((int64_t)n * a.ph + r) * a.pw + pc) * 64 + (lane >> 5) * 16;
        *reinterpret_cast<uint4*>(dst) = pk[0];
        *reinterpret_cast<uint4*>(dst + 32) = pk[1];
    };

    v16i carry[2][2], next[2][2];   // stem rows 2r-1 and 2r+1 of pooled row r
    if (r0 > 0) {                    // the band's first pooled row's upper stem row
        issue(2 * r0 - 1, kh, 0);
        IQNN_WAIT_VM_LGKM0(0);
        __builtin_amdgcn_s_barrier();
        stem_row(2 * r0 - 1, 2 * r0 - 1, 0, carry);
        __syncthreads();   // slab 0 is free again
    }
    for (int i = 0; i < kSpAhead && r0 + i < r1; ++i) issue(2 * (r0 + i), kr, (r0 + i) % kSpSlabs);
    for (int r = r0; r < r1; ++r) {
        // this pair's slab has landed (the later ones may be in flight), and every wave
        // is done with the slab refilled below
        if (r + kSpAhead - 1 < r1) {
            IQNN_WAIT_VM_LGKM0((kSpAhead - 1) * CPW);
        } else {
            IQNN_WAIT_VM_LGKM0(0);
        }
        __builtin_amdgcn_s_barrier();
        if (r + kSpAhead < r1) issue(2 * (r + kSpAhead), kr, (r + kSpAhead) % kSpSlabs);
        const int buf = r % kSpSlabs;
        v16i vm[2][2];
        stem_row(2 * r, 2 * r, buf, vm);
        if (r > 0) {   // stem row -1 lies outside the image
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int q = 0; q < 16; ++q) vm[b][t][q] = max(vm[b][t][q], carry[b][t][q]);
        }
        stem_row(2 * r + 1, 2 * r, buf, next);   // row 2r+1 < OH: OH is even
        // columns 2c-1 (block 0), 2c (block 1) and 2c+1 (block 0 of the next lane)
        int32_t h[2][16];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int32_t v0 = max(vm[0][t][q], next[0][t][q]);
                const int32_t v1 = max(vm[1][t][q], next[1][t][q]);
                h[t][q] = max(max(v0, v1), __shfl_down(v0, 1, 64));
            }
        uint4 pk[2];
        requant(h, pk);
        if (store) put(r, pk);
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int t = 0; t < 2; ++t) carry[b][t] = next[b][t];
    }
    // no DMA may still be writing this workgroup's LDS when it ends
    IQNN_WAIT_VM(0);
}

}  // namespace

// The fused stem + pooling kernel's conditions: the stem's 4-channel gather with 8-tap
// rows, stride 2 and at most kStemKH filter rows; 64 output channels of an 8-bit type
// with a requantizing Conv / Conv_Relu epilogue; an even input width (8-byte aligned
// slab reads); an even stem output height and width (pooled size = half the stem size,
// so only the window column / row -1 leaves the image); a pooled width of at most
// kSpMaxWaves * 31 columns; the input rows of a stem row pair within one slab buffer;
// and an input of whole 16-byte units (the slab DMA moves 16 bytes per lane) below 2 GB
// (32-bit offsets).
bool stem_pool_ok(const ConvParams& p) {
    if (p.kw != 8 || p.sh != 2 || p.sw != 2 || p.kh < 1 || p.kh > kStemKH || p.c_out != 64 || !p.vec_store)
        return false;
    if (p.epi != E_NONE && p.epi != E_RELU) return false;
    if (p.y_type != T_UINT8 && p.y_type != T_INT8) return false;
    if (p.w_in % 2 != 0 || p.m >= ((int64_t)1 << 31) || p.oh <= 0 || p.ow <= 0) return false;
    if (p.oh % 2 != 0 || p.ow % 2 != 0 || p.ow / 2 > kSpMaxWaves * kSpColsPerWave) return false;
    const int64_t in_bytes = (p.m / ((int64_t)p.oh * p.ow)) * p.h * (int64_t)p.w_in * 4;
    if (in_bytes % 16 != 0 || in_bytes >= ((int64_t)1 << 31)) return false;
    return (int64_t)(p.kh + 2) * p.w_in * 4 + 16 <= kSpBuf;
}

hipError_t launch_stem_pool(const ConvParams& p, uint8_t* yp, hipStream_t stream) {
    if (!stem_pool_ok(p)) return hipErrorInvalidValue;
    const int64_t n_img = p.m / ((int64_t)p.oh * p.ow);
    if (n_img <= 0) return hipSuccess;
    StemPoolArgs a;
    a.yp = yp;
    a.ph = p.oh / 2;
    a.pw = p.ow / 2;
    // about 1024 workgroups in all (four per CU, the LDS limit), bands of >= 4 rows
    a.n_bands = (int)std::max<int64_t>(1, std::min<int64_t>((1024 + n_img - 1) / n_img, (a.ph + 3) / 4));
    a.band = (a.ph + a.n_bands - 1) / a.n_bands;
    a.n_bands = (a.ph + a.band - 1) / a.band;
    a.in_bytes = n_img * p.h * (int64_t)p.w_in * 4;
    const int64_t grid = n_img * a.n_bands;
    if (grid >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    const int nw = (a.pw + kSpColsPerWave - 1) / kSpColsPerWave;
    const dim3 g((unsigned)grid), b((unsigned)(64 * nw));
    // the image stem (7 filter rows, signed input codes) takes a kernel with every choice
    // fixed at compile time; other shapes the one that reads them at run time
    const int fast = (p.kh == 7 && p.x_xor == 0u) ? 1 + (int)(p.out_fix & 1u) : 0;
    switch (nw * 3 + fast) {
#define IQNN_STEM_POOL_NW(NW_)                                                                          \
    case NW_ * 3: hipLaunchKernelGGL((qconv_stem_pool<NW_, 0, true, -1>), g, b, 0, stream, p, a); break; \
    case NW_ * 3 + 1: hipLaunchKernelGGL((qconv_stem_pool<NW_, 7, false, 0>), g, b, 0, stream, p, a); break; \
    case NW_ * 3 + 2: hipLaunchKernelGGL((qconv_stem_pool<NW_, 7, false, 1>), g, b, 0, stream, p, a); break;
    IQNN_STEM_POOL_NW(1)
    IQNN_STEM_POOL_NW(2)
    IQNN_STEM_POOL_NW(3)
    IQNN_STEM_POOL_NW(4)
#undef IQNN_STEM_POOL_NW
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// The fused 1x1 pair's conditions (see qconv_pair): both 1x1, stride 1, unpadded, over
// the same pixels (below 2^31); conv_a 64 -> 256 channels with an 8-bit residual
// (Conv_Add / Conv_Add_Relu), conv_b 256 -> 64 or 128 channels (Conv / Conv_Relu);
// 8-bit activations and outputs, symmetric dense int8 weights, the binary32
// requantization.
bool pair_ok(const ConvParams& a, const ConvParams& b) {
    auto plain1x1 = [](const ConvParams& p) {
        return p.kh == 1 && p.kw == 1 && p.sh == 1 && p.sw == 1 && p.ph == 0 && p.pw == 0 && p.vec_store &&
               p.zw_red == 0 && !p.int_rq && !p.w_idx && !p.w4 && !p.f6 &&
               (p.y_type == T_INT8 || p.y_type == T_UINT8);
    };
    if (!plain1x1(a) || !plain1x1(b) || a.m != b.m || a.m <= 0 || a.m >= ((int64_t)1 << 31)) return false;
    if (a.c != kPrCa || a.c_out != kPrCb || b.c != kPrCb || (b.c_out != 64 && b.c_out != 128)) return false;
    if ((a.epi != E_ADD && a.epi != E_ADD_RELU) || (a.res_type != T_INT8 && a.res_type != T_UINT8)) return false;
    return b.epi == E_NONE || b.epi == E_RELU;
}

hipError_t launch_pair(const ConvParams& a, const ConvParams& b, hipStream_t stream) {
    if (!pair_ok(a, b)) return hipErrorInvalidValue;
    const int64_t n_tiles = (a.m + kPrBN - 1) / kPrBN;
    const int grid = (int)std::min<int64_t>(n_tiles, 512);   // two workgroups per CU, persistent
    const bool xs = a.x_xor != 0u || b.x_xor != 0u;   // signed codes on both sides: no sign flip
    if (b.c_out == 64) {
        if (xs) hipLaunchKernelGGL((qconv_pair<64, true>), dim3(grid), dim3(256), 0, stream, a, b, (int32_t)n_tiles);
        else hipLaunchKernelGGL((qconv_pair<64, false>), dim3(grid), dim3(256), 0, stream, a, b, (int32_t)n_tiles);
    } else {
        if (xs) hipLaunchKernelGGL((qconv_pair<128, true>), dim3(grid), dim3(256), 0, stream, a, b, (int32_t)n_tiles);
        else hipLaunchKernelGGL((qconv_pair<128, false>), dim3(grid), dim3(256), 0, stream, a, b, (int32_t)n_tiles);
    }
    return hipGetLastError();
}

namespace {

// ============================================================ direct 3x3 kernel
//
// qconv_direct3x3: 3x3 / stride 1 / pad 1 convolution of 64-channel 8-bit codes on rows
// of W pixels (W <= 64), as a direct convolution.  A tile is two output rows of one image
// (2W pixels, four 32-pixel MFMA blocks, one per wave; lanes past 2W compute a clamped
// pixel and store nothing).  The four input rows the tile reads -- with the input
// zero-point code in the padding, so the padded taps need no test -- are copied into
// LDS once per tile by 16-byte DMA (slab rows of W+2 pixels x 64 bytes, the four
// 16-byte slots of a pixel swizzled by bits 2-3 of its column, as the streaming
// kernel's rows).  Three slab buffers: the slab of the tile after next is issued at
// the start of a tile, two tiles ahead, and the wait for a slab leaves the newest
// stores in flight.  Every wave holds
// the A fragments of the block's 64 output channels for all K = 9 x 64 in registers
// and reads its B fragment of tap (ky, kx), k-step ks straight from the slab: the
// implicit GEMM's nine reads of every input row from L2 become one, and no weight
// bytes move per tile.
// OUTK: the epilogue's output kind (1 = 8-bit codes, 2 = raw int32, 3 = 4-bit codes).
constexpr int kD3Buf = 16384;   // LDS bytes per slab buffer (4 rows of up to 62 pixels)
constexpr int64_t kD3MinTiles = 512;

// SP: 2:4-sparse weights (one tap of 64 input channels is one 64-K stage of the 2:4
// blocks): per channel block and tap a 16-byte fragment of kept codes and its 32-bit
// positions in registers, one sparse MFMA per tap on the tap's two k-step fragments.
template <int W, int OUTK, bool XORB, bool INTRQ = false, bool SP = false>
__global__ __launch_bounds__(256, 2) void qconv_direct3x3(const ConvParams p, int32_t n_tiles,
                                                           int32_t tiles_per_img) {
    constexpr int SW = W + 2;                       // slab columns: one pad column each side
    constexpr int CHUNKS = 4 * SW * 4;              // 16-byte chunks of the four slab rows
    constexpr int CPW = (CHUNKS + 255) / 256;       // DMA instructions per wave (64 chunks each)
    static_assert(W % 2 == 0 && 2 * W <= 128, "two rows are at most four 32-pixel blocks");
    static_assert(CPW * 4 * 1024 <= kD3Buf, "a slab fits one buffer");
    __shared__ __attribute__((aligned(1024))) uint8_t slab[3][kD3Buf];
    __shared__ __attribute__((aligned(16))) int32_t cbias[64];
    __shared__ __attribute__((aligned(16))) float cmult[64];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int oc0 = (int)blockIdx.y * 64;
    if ((int)blockIdx.x >= n_tiles) return;
    if (tid < 64) {
        cbias[tid] = p.bias[oc0 + tid];
        cmult[tid] = p.mult[oc0 + tid];
    }
    // A fragments: packed rows oc0 + 32t + lane%32, K bytes 64 tap + 32 ks + 16 (lane/32);
    // 2:4 weights: that row's kept codes of K half lane/32 of stage `tap` and their
    // positions, from the (128-row tile, stage) block
    v4i wa[2][9][SP ? 1 : 2];
    int wix[SP ? 2 : 1][SP ? 9 : 1];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int tap = 0; tap < 9; ++tap) {
            const int row = oc0 + 32 * t + (lane & 31);
            if constexpr (SP) {
                const int rr = row % kSpRows, hh = lane >> 5;
                const int8_t* blk = p.w + ((int64_t)(row / kSpRows) * (p.kp / kPipeBK) + tap) * kSpBlock;
                wa[t][tap][0] = *reinterpret_cast<const v4i*>(blk + rr * 32 + ((hh ^ ((rr >> 3) & 1)) * 16));
                wix[t][tap] = *reinterpret_cast<const int*>(blk + kSpRows * 32 + rr * 8 + hh * 4);
            } else {
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    wa[t][tap][ks] = *reinterpret_cast<const v4i*>(p.w + (int64_t)row * p.kp + 64 * tap + 32 * ks +
                                                                   16 * (lane >> 5));
            }
        }
    __syncthreads();
    // integer-only requantization: the binary32 evaluation when every multiplier of the
    // block's output channels is at least 2^-13 (see epi_store16)
    bool irq32 = false;
    if constexpr (INTRQ) irq32 = __all(oc0 + lane >= p.c_out || cmult[lane] >= 0x1p-13f) != 0;

    const int h = p.h;
    // Chunk q = (wave + 4j) * 64 + lane of a slab buffer (its bytes 16q..16q+15) is slab
    // row q / (4 SW), column (q / 4) % SW, slot q % 4, and holds channel chunk
    // slot ^ ((column >> 2) & 3) of input row oy0 - 1 + row, column - 1.  Per lane and DMA
    // instruction j, fixed for the whole launch: the chunk's byte offset from the start
    // of input row oy0 - 1, and its slab row minus one (iy - oy0), or a row no image has
    // for the pad columns and the chunks past the slab.
    int loff[CPW], rm1[CPW];
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
        const int q = (wave + 4 * j) * 64 + lane;   // < 4 * CPW * 64: inside the buffer
        const int row = q / (SW * 4), rem = q - row * (SW * 4);
        const int col = rem >> 2, slot = rem & 3;
        const int chunk = slot ^ ((col >> 2) & 3);
        const bool in_img_col = q < CHUNKS && col >= 1 && col <= W;
        loff[j] = in_img_col ? (row * W + col - 1) * 64 + chunk * 16 : 0;
        rm1[j] = in_img_col ? row - 1 : (1 << 30);   // h < 2^31 / 56 < 2^30
    }
    // Slab of tile `tile` into buffer `buf`: every lane issues its CPW DMA instructions
    // (the waits count them), from the input where the chunk's row and column are in the
    // image and from the 16 pad-code bytes of pad_row elsewhere.  Tiles never exceed the
    // batch, so in-image rows and columns stay inside the n x h x W x 64 input.
    auto issue = [&](int tile, int buf) {
        const int n = tile / tiles_per_img;
        const int oy0 = 2 * (tile - n * tiles_per_img);
        const int64_t row0 = ((int64_t)n * h + oy0 - 1) * W * 64;   // input row oy0 - 1
#pragma unroll
        for (int j = 0; j < CPW; ++j) {
            const void* src = (uint32_t)(oy0 + rm1[j]) < (uint32_t)h ? (const void*)(p.x + (row0 + loff[j]))
                                                                     : (const void*)p.pad_row;
            dma16_run<1>(lds_addr(&slab[buf][0]) + (wave + 4 * j) * 1024, &src);
        }
    };

    const int frow = lane & 31;
    const int i = min(wave * 32 + frow, 2 * W - 1);   // pixel of the row pair
    const int r = i >= W ? 1 : 0, ox = i - r * W;
    const bool px_ok = wave * 32 + frow < 2 * W;
    const uint32_t bxor = XORB ? p.x_xor : 0u;
    const int grid = (int)gridDim.x;
    // this lane's fragment offset inside a slab for filter column kx and k-step ks (the
    // filter row adds ky * SW * 64, a constant), fixed for the launch
    int boff[3][2];
#pragma unroll
    for (int kx = 0; kx < 3; ++kx)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int col = ox + kx;
            boff[kx][ks] = (r * SW + col) * 64 + (((2 * ks + (lane >> 5)) ^ ((col >> 2) & 3)) << 4);
        }
    issue(blockIdx.x, 0);
    if ((int)blockIdx.x + grid < n_tiles) issue(blockIdx.x + grid, 1);
    bool stored = false;   // this wave issued the (at least two) stores of its previous tile
    // one tile in slab buffer BUF (a compile-time constant: the tiles of a workgroup take
    // the three buffers in turn, so the loop below runs in rounds of three)
    auto tile_body = [&](auto buf_c, int tile) {
        constexpr int buf = decltype(buf_c)::value;
        // The memory counter retires loads and stores in issue order, so vmcnt <= N
        // means all but the newest N operations are done.  Issued after this tile's
        // slab: the next tile's slab (CPW DMA, if there is a next tile), the previous
        // tile's stores (two or more, if any lane had a pixel) and possibly older stores:
        // N = CPW + 2 waits for the slab and never for the newest stores.
        if (tile + grid < n_tiles) {
            if (stored) IQNN_WAIT_VM(CPW + 2);
            else IQNN_WAIT_VM(CPW);
        } else {
            if (stored) IQNN_WAIT_VM(2);
            else IQNN_WAIT_VM(0);
        }
        // every wave's part of the slab has landed, and every wave is done with the
        // previous tile's buffer, which takes the slab of the tile after next
        __builtin_amdgcn_s_barrier();
        {
            const int after = tile + 2 * grid;
            if (after < n_tiles) issue(after, (buf + 2) % 3);
        }

        v16i acc[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int ocl = t * 32 + (lane >> 5) * 16;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int4 bv = *reinterpret_cast<const int4*>(&cbias[ocl + 4 * q]);
                acc[t][4 * q] = bv.x; acc[t][4 * q + 1] = bv.y; acc[t][4 * q + 2] = bv.z; acc[t][4 * q + 3] = bv.w;
            }
        }
        // B fragment s = (tap, k-step) of this lane's pixel, read one step ahead of its
        // two MFMAs (a scheduling barrier per step keeps the reads from piling up in
        // registers next to the A fragments)
        auto read_b = [&](int s) -> v4i {
            const int tap = s >> 1, ks = s & 1;
            const int ky = tap / 3, kx = tap - 3 * ky;
            return *reinterpret_cast<const v4i*>(&slab[buf][ky * SW * 64] + boff[kx][ks]);
        };
        if constexpr (SP) {
            // one tap per step: its two k-step fragments are the sparse MFMA's B operand
            v4i f0 = read_b(0), f1 = read_b(1);
#pragma unroll
            for (int tap = 0; tap < 9; ++tap) {
                v4i n0, n1;
                if (tap + 1 < 9) {
                    n0 = read_b(2 * tap + 2);
                    n1 = read_b(2 * tap + 3);
                }
                if constexpr (XORB) {
                    f0[0] ^= bxor; f0[1] ^= bxor; f0[2] ^= bxor; f0[3] ^= bxor;
                    f1[0] ^= bxor; f1[1] ^= bxor; f1[2] ^= bxor; f1[3] ^= bxor;
                }
                const v8i fb8 = {f0[0], f0[1], f0[2], f0[3], f1[0], f1[1], f1[2], f1[3]};
                acc[0] = __builtin_amdgcn_smfmac_i32_32x32x64_i8(wa[0][tap][0], fb8, acc[0], wix[0][tap], 0, 0);
                acc[1] = __builtin_amdgcn_smfmac_i32_32x32x64_i8(wa[1][tap][0], fb8, acc[1], wix[1][tap], 0, 0);
                __builtin_amdgcn_sched_barrier(0);
                if (tap + 1 < 9) {
                    f0 = n0;
                    f1 = n1;
                }
            }
        } else {
            v4i fb = read_b(0);
#pragma unroll
            for (int s = 0; s < 18; ++s) {
                v4i fn;
                if (s + 1 < 18) fn = read_b(s + 1);
                if constexpr (XORB) {
                    fb[0] ^= bxor; fb[1] ^= bxor; fb[2] ^= bxor; fb[3] ^= bxor;
                }
                acc[0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(wa[0][s >> 1][s & 1], fb, acc[0], 0, 0, 0);
                acc[1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(wa[1][s >> 1][s & 1], fb, acc[1], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
                if (s + 1 < 18) fb = fn;
            }
        }
        const int n = tile / tiles_per_img;
        const int oy = 2 * (tile - n * tiles_per_img) + r;
        const bool st = px_ok && oy < h;
        stored = __builtin_amdgcn_ballot_w64(st) != 0;
        if (st) {
            const int64_t pix = ((int64_t)n * h + oy) * W + ox;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int ocl = t * 32 + (lane >> 5) * 16;
                if (oc0 + ocl >= p.c_out) continue;
                uint32_t rw[4] = {0, 0, 0, 0};
                // multipliers read from LDS inside the epilogue: no register copy next to
                // the 144 registers of A fragments
                epi_store16<false, 2, INTRQ, OUTK>(p, acc[t], nullptr, &cmult[ocl], rw, oc0 + ocl, pix, false,
                                                   0.0f, irq32);
            }
        }
    };
    for (int tile = blockIdx.x; tile < n_tiles;) {
        tile_body(std::integral_constant<int, 0>{}, tile);
        if ((tile += grid) >= n_tiles) break;
        tile_body(std::integral_constant<int, 1>{}, tile);
        if ((tile += grid) >= n_tiles) break;
        tile_body(std::integral_constant<int, 2>{}, tile);
        tile += grid;
    }
    // no DMA may still be writing this workgroup's LDS when it ends
    IQNN_WAIT_VM(0);
}

}  // namespace

// The direct 3x3 kernel's conditions: 8-bit activations with 64 channels, 3x3 / stride 1
// / pad 1 on rows of 56 pixels (the instantiated width), C_out % 64 == 0, no residual,
// the binary32 requant without the weight zero-point term.  The automatic choice also
// asks for at least one two-row tile per workgroup slot (N x ceil(H / 2) >= 512), so
// the per-workgroup weight load pays off.
bool direct3x3_ok(const ConvParams& p, int gather, bool forced) {
    if (gather != GATHER_B8 || p.c != 64 || p.kh != 3 || p.kw != 3 || p.sh != 1 || p.sw != 1) return false;
    if (p.ph != 1 || p.pw != 1 || p.w_in != 56 || p.ow != 56 || p.oh != p.h) return false;
    if (p.c_out % 64 != 0 || p.epi == E_ADD || p.epi == E_ADD_RELU || p.zw_red != 0) return false;
    if (p.int_rq && p.y_type != T_INT8 && p.y_type != T_UINT8) return false;   // 8-bit codes only
    if (p.w_idx && p.epi != E_RAW && p.y_type != T_INT8 && p.y_type != T_UINT8) return false;
    if (p.m >= ((int64_t)1 << 31)) return false;
    return forced || (p.m / ((int64_t)p.oh * p.ow)) * ((p.oh + 1) / 2) >= kD3MinTiles;
}

hipError_t launch_direct3x3(const ConvParams& p, hipStream_t stream) {
    const int64_t n_img = p.m / ((int64_t)p.oh * p.ow);
    const int64_t tiles_per_img = (p.oh + 1) / 2;
    const int64_t n_tiles = n_img * tiles_per_img;
    if (n_tiles <= 0) return hipSuccess;
    if (n_tiles >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    const int64_t oc_blocks = p.c_out / 64;
    const int64_t per_block = std::min<int64_t>(n_tiles, std::max<int64_t>(1, 512 / oc_blocks));   // ~2 per CU
    const dim3 grid((unsigned)per_block, (unsigned)oc_blocks);
    const int32_t nt = (int32_t)n_tiles, tpi = (int32_t)tiles_per_img;
    // signed activation codes are MFMA operands as they are; uint8 ones get the sign flip
    const bool xorb = p.x_xor != 0;
    if (p.w_idx) {   // 2:4 weights: 8-bit codes or raw int32
        if (p.epi == E_RAW) {
            if (xorb) hipLaunchKernelGGL((qconv_direct3x3<56, 2, true, false, true>), grid, dim3(256), 0, stream, p, nt, tpi);
            else hipLaunchKernelGGL((qconv_direct3x3<56, 2, false, false, true>), grid, dim3(256), 0, stream, p, nt, tpi);
        } else {
            if (xorb) hipLaunchKernelGGL((qconv_direct3x3<56, 1, true, false, true>), grid, dim3(256), 0, stream, p, nt, tpi);
            else hipLaunchKernelGGL((qconv_direct3x3<56, 1, false, false, true>), grid, dim3(256), 0, stream, p, nt, tpi);
        }
    } else if (p.int_rq) {   // integer-only requantization to 8-bit codes
        if (xorb) hipLaunchKernelGGL((qconv_direct3x3<56, 1, true, true>), grid, dim3(256), 0, stream, p, nt, tpi);
        else hipLaunchKernelGGL((qconv_direct3x3<56, 1, false, true>), grid, dim3(256), 0, stream, p, nt, tpi);
    } else if (p.epi == E_RAW) {
        if (xorb) hipLaunchKernelGGL((qconv_direct3x3<56, 2, true>), grid, dim3(256), 0, stream, p, nt, tpi);
        else hipLaunchKernelGGL((qconv_direct3x3<56, 2, false>), grid, dim3(256), 0, stream, p, nt, tpi);
    } else if (p.y_type == T_INT8 || p.y_type == T_UINT8) {
        if (xorb) hipLaunchKernelGGL((qconv_direct3x3<56, 1, true>), grid, dim3(256), 0, stream, p, nt, tpi);
        else hipLaunchKernelGGL((qconv_direct3x3<56, 1, false>), grid, dim3(256), 0, stream, p, nt, tpi);
    } else {
        if (xorb) hipLaunchKernelGGL((qconv_direct3x3<56, 3, true>), grid, dim3(256), 0, stream, p, nt, tpi);
        else hipLaunchKernelGGL((qconv_direct3x3<56, 3, false>), grid, dim3(256), 0, stream, p, nt, tpi);
    }
    return hipGetLastError();
}

bool pipe_eligible(int gather, int32_t c, int64_t k) {
    return (gather == GATHER_B8 && c % 64 == 0 && k % kPipeBK == 0) || gather == GATHER_C4;
}

// Tile configurations of the pipelined kernel (block channels x pixels, waves along
// channels, ring depth).
using P64x256 = PipeCfg<64, 256, 1, 4>;
using P128x128 = PipeCfg<128, 128, 2, 4>;
using P128x256 = PipeCfg<128, 256, 2, 3>;
using P256x128 = PipeCfg<256, 128, 2, 3>;
using P256x256 = PipeCfg<256, 256, 2, 4>;
using P128x128s3 = PipeCfg<128, 128, 2, 3>;
using P64x128 = PipeCfg<64, 128, 1, 4>;
using S64x128d12 = StreamCfg<64, 128, 1, 12>;
using S64x128d6 = StreamCfg<64, 128, 1, 6>;
using S128x128d8 = StreamCfg<128, 128, 2, 8>;
using S128x128d4 = StreamCfg<128, 128, 2, 4>;
using S128x128w1d4 = StreamCfg<128, 128, 1, 4>;
using S64x256d3 = StreamCfg<64, 256, 1, 3>;
using S256x128d6 = StreamCfg<256, 128, 2, 6>;
using S128x256d6 = StreamCfg<128, 256, 2, 6>;
using S128x128d3o3 = StreamCfg<128, 128, 2, 3, 3>;
using S128x256d3 = StreamCfg<128, 256, 2, 3>;
using S256x128d3 = StreamCfg<256, 128, 2, 3>;
using S256x256d4 = StreamCfg<256, 256, 2, 4>;
// eight waves per workgroup, one workgroup per CU (each wave 128 channels x 64 or 32 pixels)
using W256x256d4 = StreamCfg<256, 256, 2, 4, 1, kPipeBK, 8>;
using W128x512d3 = StreamCfg<128, 512, 1, 3, 1, kPipeBK, 8>;
using W256x128d4 = StreamCfg<256, 128, 2, 4, 1, kPipeBK, 8>;
using W512x128d3 = StreamCfg<512, 128, 4, 3, 1, kPipeBK, 8>;

// the block configurations the automatic tile choice makes for layers without a
// residual (tiles 8, 10, 11, 14, 16 and 22) carry the integer-only requantization
template <> constexpr bool kIrqTile<S64x128d6> = true;
template <> constexpr bool kIrqTile<S128x128d4> = true;
template <> constexpr bool kIrqTile<S64x256d3> = true;
template <> constexpr bool kIrqTile<S256x128d3> = true;
template <> constexpr bool kIrqTile<S128x128d3o3> = true;
template <> constexpr bool kIrqTile<W256x128d4> = true;

// Automatic tile (per-layer sweeps over the trunk's shapes at batch 256 chose these),
// mostly on the streaming kernel at two blocks per CU: 256x128 blocks
// (each wave 128 channels x 64 pixels: 0.75 KB of fragment reads per MFMA) for the
// wide, deep contractions (C_out >= 256, K >= 1024, no residual); 128x128 blocks
// for the rest.  C_out <= 64: 64x256 blocks (each wave 64 x 64: 1 KB of fragment
// reads per MFMA, 20 KB stages at ring depth 3) for one-stage and 3x3-deep
// contractions, 64x128 blocks (deeper ring) between those.  Without a residual and
// with C_out >= 128, the very deep contractions (K >= 4096) and the one-stage ones
// run 128x128 blocks three to a CU, and C_out >= 512 takes the 256x128 blocks at any K.
int pipe_tile_choice(int64_t m, int32_t c_out, int64_t k, bool res) {
    (void)m;
    // very deep contractions of 512+ channels: one 8-wave 256x128 block per CU
    if (!res && c_out >= 512 && k >= 4096) return 22;
    if (!res && c_out >= 128 && (k >= 4096 || k == kPipeBK)) return 14;
    // 128-channel contractions of at least 1024: 128x128 blocks three to a CU
    if (!res && c_out == 128 && k >= 1024) return 14;
    if (!res && c_out >= 256 && (k >= 1024 || c_out >= 512)) return 16;
    if (c_out <= 64) return (k == kPipeBK || k >= 576) ? 11 : 8;
    return 10;
}

hipError_t launch_qconv(const ConvParams& p, int gather, bool is_1x1, hipStream_t stream, int tile) {
    if (p.f6 && gather != GATHER_B4S) return hipErrorInvalidValue;
    if (tile == kTileFp6) tile = -1;   // the FP6 path is chosen by the host (ConvParams::f6)
    if (p.w_idx) {   // 2:4 weights: their packed layout is the sparse streaming kernel's
        const bool add = p.epi == E_ADD || p.epi == E_ADD_RELU;
        const bool res_prefetch = add && p.vec_store && (p.res_type == T_INT8 || p.res_type == T_UINT8);
        if (gather != GATHER_B8 || !pipe_eligible(gather, p.c, p.k) || p.zw_red != 0 || (add && !res_prefetch))
            return hipErrorInvalidValue;
        if (direct3x3_ok(p, gather, tile == kTileDirect3x3)) return launch_direct3x3(p, stream);
        return launch_stream_2of4(p, is_1x1, stream);
    }
    if (tile == kTileDirect3x3) {   // the direct kernel where it applies, else the automatic choice
        if (direct3x3_ok(p, gather, true)) return launch_direct3x3(p, stream);
        tile = -1;
    }
    if (tile < 0 && direct3x3_ok(p, gather, false)) return launch_direct3x3(p, stream);
    if (p.int_rq) {   // integer-only requantization: the streaming kernel, else the register-staged one
        if (p.zw_red != 0) return hipErrorInvalidValue;
        const bool out8 = (p.y_type == T_INT8 || p.y_type == T_UINT8) && p.vec_store;
        if (gather == GATHER_B8 && out8 && pipe_eligible(gather, p.c, p.k) && p.m < ((int64_t)1 << 31) &&
            (is_1x1 || p.kh * p.kw <= 64)) {
            // the automatic choice (an explicit tile without the integer variant takes it too)
            const int t = (tile == 8 || tile == 10 || tile == 11 || tile == 14 || tile == 16 || tile == 22)
                              ? tile : pipe_tile_choice(p.m, p.c_out, p.k, false);
            switch (t) {
            case 14: return launch_stream<S128x128d3o3>(p, is_1x1, false, false, stream);
            case 8: return launch_stream<S64x128d6>(p, is_1x1, false, false, stream);
            case 10: return launch_stream<S128x128d4>(p, is_1x1, false, false, stream);
            case 11: return launch_stream<S64x256d3>(p, is_1x1, false, false, stream);
            case 16: return launch_stream<S256x128d3>(p, is_1x1, false, false, stream);
            default: return launch_stream<W256x128d4>(p, is_1x1, false, false, stream);
            }
        }
        if (p.c_out <= 64) return launch_staged<64, 256, 1, 4>(p, gather, is_1x1, stream);
        return launch_staged<128, 128, 2, 2>(p, gather, is_1x1, stream);
    }
    if (gather == GATHER_C4 && tile < 0 && stem_ok(p)) return launch_stem(p, stream);
    if (gather == GATHER_B4S) {   // its packed layout is the streaming kernel's: no other tile
        if (p.c_out <= 64)
            return p.f6 ? launch_stream_b4<S64x128d6, true>(p, is_1x1, stream)
                        : launch_stream_b4<S64x128d6, false>(p, is_1x1, stream);
        // FP6: one wave per 128 channels x 32 pixels, so each activation fragment turned
        // into BF6 feeds four MFMAs
        if (p.f6) return launch_stream_b4<S128x128w1d4, true>(p, is_1x1, stream);
        return launch_stream_b4<S128x128d4, false>(p, is_1x1, stream);
    }
    if (p.zw_red != 0) {   // asymmetric weights ride on the streaming kernel only
        const bool add = p.epi == E_ADD || p.epi == E_ADD_RELU;
        const bool res_prefetch = add && p.vec_store && (p.res_type == T_INT8 || p.res_type == T_UINT8);
        if (gather != GATHER_B8 || !pipe_eligible(gather, p.c, p.k) || (add && !res_prefetch))
            return hipErrorInvalidValue;
        if (p.c_out <= 64) return launch_stream<S64x256d3>(p, is_1x1, res_prefetch, false, stream, true);
        return launch_stream<S128x128d4>(p, is_1x1, res_prefetch, false, stream, true);
    }
    if (pipe_eligible(gather, p.c, p.k)) {
        const bool c4 = gather == GATHER_C4;
        const bool add = p.epi == E_ADD || p.epi == E_ADD_RELU;
        const bool res_prefetch = add && p.vec_store && (p.res_type == T_INT8 || p.res_type == T_UINT8);
        if (tile < 0) tile = pipe_tile_choice(p.m, p.c_out, p.k, res_prefetch);
        // eight-wave blocks stream neither a residual stage nor the 4-channel gather
        if (tile >= 20 && (add || c4)) tile = p.c_out <= 64 ? 11 : 10;
        // 512-channel blocks need C_out padded to 256 to be a multiple of 512
        if (tile == 23 && !block_fits_packed(p.c_out, 512)) tile = 20;
        // the streaming kernel takes a residual only as a stage of its stream, decodes
        // pixel indices in 32 bits and keeps a 64-bit mask of in-image filter taps
        const bool stream_ok = p.m < ((int64_t)1 << 31) && (is_1x1 || c4 || p.kh * p.kw <= 64);
        if (tile == 14 && (add || c4)) tile = 10;   // compiled without those variants
        if (tile >= 7 && (!stream_ok || (add && !(res_prefetch && tile != 12 && tile != 13 && tile < 15))))
            tile = p.c_out <= 64 ? 0 : 1;
        if (c4 && tile >= 7 && tile != 8 && tile != 10 && tile != 12) tile = p.c_out <= 64 ? 8 : 10;
        if (c4 && tile < 7 && tile != 0 && tile != 1 && tile != 6) tile = p.c_out <= 64 ? 0 : 1;   // the 4-channel gather's shapes
        switch (tile) {
        case 0: return launch_pipe<P64x256>(p, is_1x1, res_prefetch, c4, stream);
        case 1: return launch_pipe<P128x128>(p, is_1x1, res_prefetch, c4, stream);
        case 2: return launch_pipe<P128x256>(p, is_1x1, res_prefetch, c4, stream);
        case 3: return launch_pipe<P256x128>(p, is_1x1, res_prefetch, c4, stream);
        case 4: return launch_pipe<P256x256>(p, is_1x1, res_prefetch, c4, stream);
        case 5: return launch_pipe<P128x128s3>(p, is_1x1, res_prefetch, c4, stream);
        case 6: return launch_pipe<P64x128>(p, is_1x1, res_prefetch, c4, stream);
        case 7: return launch_stream<S64x128d12>(p, is_1x1, res_prefetch, c4, stream);
        case 8: return launch_stream<S64x128d6>(p, is_1x1, res_prefetch, c4, stream);
        case 9: return launch_stream<S128x128d8>(p, is_1x1, res_prefetch, c4, stream);
        case 10: return launch_stream<S128x128d4>(p, is_1x1, res_prefetch, c4, stream);
        case 11: return launch_stream<S64x256d3>(p, is_1x1, res_prefetch, c4, stream);
        case 12: return launch_stream<S256x128d6>(p, is_1x1, res_prefetch, c4, stream);
        case 13: return launch_stream<S128x256d6>(p, is_1x1, res_prefetch, c4, stream);
        case 14: return launch_stream<S128x128d3o3>(p, is_1x1, res_prefetch, c4, stream);
        case 15: return launch_stream<S128x256d3>(p, is_1x1, res_prefetch, c4, stream);
        case 16: return launch_stream<S256x128d3>(p, is_1x1, res_prefetch, c4, stream);
        case 17: return launch_stream<S256x256d4>(p, is_1x1, res_prefetch, c4, stream);
        case 20: return launch_stream<W256x256d4>(p, is_1x1, res_prefetch, c4, stream);
        case 21: return launch_stream<W128x512d3>(p, is_1x1, res_prefetch, c4, stream);
        case 22: return launch_stream<W256x128d4>(p, is_1x1, res_prefetch, c4, stream);
        default: return launch_stream<W512x128d3>(p, is_1x1, res_prefetch, c4, stream);
        }
    }
    if (p.c_out <= 64) return launch_staged<64, 256, 1, 4>(p, gather, is_1x1, stream);
    return launch_staged<128, 128, 2, 2>(p, gather, is_1x1, stream);
}

}  // namespace iqnn
