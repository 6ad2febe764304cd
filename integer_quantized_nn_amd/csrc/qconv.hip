// qconv.hip -- implicit-GEMM quantized convolution / GEMM for gfx950 (CDNA4).
//
// The operator (MegEngine 4-bit article, sections 緩解精度下降, 算子融合優化 and
// conv 算子優化; "Quantization" blog, section 量化矩阵乘):
//   acc[p][oc] = sum_k A[p][k] * W[oc][k]            int8 x int8 -> int32 (MFMA)
//   a          = acc + bias_fold[oc]                  zero-point terms folded in
//   y[p][oc]   = epilogue(a)                          requant / ReLU / residual add
// where p runs over output pixels (n, oh, ow) and k over (kh, kw, ci).  The im2col
// matrix A is never built: each workgroup gathers its tile straight from the NHWC
// activations while staging it into LDS, as the MegEngine article describes for
// its global->shared load (conv 算子優化, after Fig. 5).
//
// gfx950 design
//   * Contraction on v_mfma_i32_16x16x64_i8 (signed int8 only).  UINT8 activations
//     are shifted to int8 with XOR 0x80 during staging (q - 128); the host folds
//     the +128*sum(W) back into the bias.  4-bit activations are unpacked to int8
//     during staging (UINT4 zero-extended, INT4 sign-extended): CDNA4 has no 4-bit
//     integer MFMA, so 4-bit data saves HBM bytes, not MFMA cycles.
//   * The output channel is the MFMA row (A operand = weights) and the pixel the
//     MFMA column (B operand = activations), so the accumulator a lane holds runs
//     along channels -- the NHWC-friendly orientation the MegEngine article gets by
//     transposing its output (conv 算子優化, Fig. 7 and after).  The prepacked
//     weight rows are permuted (the column-permutation identity of its Fig. 8) so
//     each lane ends with 16 consecutive channels: one 16-byte store per pixel.
//   * 256 threads = 4 waves; each wave owns 64 channels x (BN/WN) pixels.  K is
//     staged 128 elements at a time through double-buffered LDS with rows padded
//     to 144 bytes, which keeps the 16-byte fragment reads bank-conflict free.
//   * Workgroup ids are remapped so that consecutive tiles land on the same XCD
//     (workgroups are dealt round-robin over the 8 XCDs, each with its own L2).
//   * The epilogue runs in registers in strict binary32 (no contraction), with
//     round-half-to-even, then packs and stores.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "iqnn_internal.h"

#pragma clang fp contract(off)

namespace iqnn {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kLdsStride = kBK + 16;   // bytes per staged row
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

// One requantized output, strict binary32, one rounding per operation.
__device__ __forceinline__ int32_t requant_one(int32_t a, float m, int32_t rcode, bool add, bool relu,
                                               float m_res, const ConvParams& p) {
    float t = (float)a * m;
    if (add) {
        float d = (float)(rcode - p.z_res);
        float u = d * m_res;
        t = t + u;
    }
    if (relu) t = (t > 0.0f) ? t : 0.0f;
    float r = __builtin_rintf(t);
    r = fminf(fmaxf(r, p.lo), p.hi);
    return (int32_t)r + p.z_out;
}

__device__ __forceinline__ int32_t res_code(const uint32_t* rw, int i, int type) {
    if (type == T_UINT8) return (int32_t)((rw[i >> 2] >> (8 * (i & 3))) & 0xFF);
    if (type == T_INT8) return (int32_t)(int8_t)((rw[i >> 2] >> (8 * (i & 3))) & 0xFF);
    int32_t nib = (int32_t)((rw[i >> 3] >> (4 * (i & 7))) & 0xF);
    if (type == T_INT4 && nib >= 8) nib -= 16;
    return nib;
}

// The second launch bound is the number of workgroups per CU that the LDS
// footprint allows (160 KB of LDS per CU on gfx950).
template <int BM, int BN, int WM, int WN, int GATHER, bool IS1X1>
__global__ __launch_bounds__(256, (2 * 2 * (BM + BN) * kLdsStride <= 160 * 1024 ? 2 : 1))
void qconv_igemm(const ConvParams p) {
    constexpr int WPX = BN / WN;      // pixels per wave
    constexpr int TN = WPX / 16;      // MFMA tiles along pixels per wave
    constexpr int A_SEGS = BM * kSegPerRow / 256;
    constexpr int B_SEGS = BN * kSegPerRow / 256;
    static_assert(BM / WM == 64, "a wave owns 64 output channels");
    static_assert(WM * WN == 4, "four waves");
    static_assert(A_SEGS >= 1 && B_SEGS >= 1, "tile too small");

    __shared__ __attribute__((aligned(16))) uint8_t lds[2][(BM + BN) * kLdsStride];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wave_oc = wave % WM;
    const int wave_px = wave / WM;

    // XCD-aware remap of the workgroup id: the hardware deals ids round-robin over
    // 8 XCDs; give each XCD a contiguous range of logical tiles.
    const int G = gridDim.x;
    const int bid = blockIdx.x;
    const int xcd = bid & 7, idx = bid >> 3;
    const int q8 = G >> 3, r8 = G & 7;
    const int L = (xcd < r8) ? xcd * (q8 + 1) + idx : r8 * (q8 + 1) + (xcd - r8) * q8 + idx;
    const int tile_oc = L % p.n_oc_tiles;
    const int tile_px = L / p.n_oc_tiles;
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

    v4i acc[4][TN];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int u = 0; u < TN; ++u) acc[t][u] = v4i{0, 0, 0, 0};

    const int nstages = (p.kp + kBK - 1) / kBK;
    const int frag_row = lane & 15;
    const int frag_col = (lane >> 4) * 16;
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
        for (int kk = 0; kk < kBK / 64; ++kk) {
            if (s * kBK + kk * 64 >= p.kp) break;
            v4i a[4], b[TN];
#pragma unroll
            for (int t = 0; t < 4; ++t)
                a[t] = *reinterpret_cast<const v4i*>(&L0[(a_row0 + t * 16) * kLdsStride + kk * 64 + frag_col]);
#pragma unroll
            for (int u = 0; u < TN; ++u)
                b[u] = *reinterpret_cast<const v4i*>(&L0[(b_row0 + u * 16) * kLdsStride + kk * 64 + frag_col]);
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int u = 0; u < TN; ++u)
                    acc[t][u] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[t], b[u], acc[t][u], 0, 0, 0);
        }
        if (more) store_stage(buf ^ 1);
        __syncthreads();
    }

    // ---------------------------------------------------------------- epilogue
    // Lane group g holds MFMA rows 4g..4g+3 of each of the 4 channel tiles; with the
    // packed row permutation these are physical channels ocb + 4t + r.
    const int g = lane >> 4;
    const int ocb = oc0 + wave_oc * 64 + g * 16;
    if (ocb >= p.c_out) return;
    const bool add = p.epi == E_ADD || p.epi == E_ADD_RELU;
    const bool relu = p.epi == E_RELU || p.epi == E_ADD_RELU;
    const float m_res = add ? *p.m_res : 0.0f;

    int32_t bias[16];
    float mult[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        int4 bv = *reinterpret_cast<const int4*>(p.bias + ocb + 4 * j);
        float4 mv = *reinterpret_cast<const float4*>(p.mult + ocb + 4 * j);
        bias[4 * j] = bv.x; bias[4 * j + 1] = bv.y; bias[4 * j + 2] = bv.z; bias[4 * j + 3] = bv.w;
        mult[4 * j] = mv.x; mult[4 * j + 1] = mv.y; mult[4 * j + 2] = mv.z; mult[4 * j + 3] = mv.w;
    }

#pragma unroll
    for (int u = 0; u < TN; ++u) {
        const int64_t pix = px0 + wave_px * WPX + u * 16 + frag_row;
        if (pix >= p.m) continue;
        int32_t a[16];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) a[4 * t + r] = acc[t][u][r] + bias[4 * t + r];

        const int64_t oidx = pix * p.c_out + ocb;   // element index of the first channel
        if (p.epi == E_RAW) {
            int32_t* yo = reinterpret_cast<int32_t*>(p.y) + oidx;
            if (p.vec_store) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    *reinterpret_cast<int4*>(yo + 4 * j) = make_int4(a[4 * j], a[4 * j + 1], a[4 * j + 2], a[4 * j + 3]);
            } else {
                for (int j = 0; j < 16 && ocb + j < p.c_out; ++j) yo[j] = a[j];
            }
            continue;
        }

        uint32_t rw[4] = {0, 0, 0, 0};
        if (add) {
            if (p.res_type == T_INT8 || p.res_type == T_UINT8) {
                if (p.vec_store) {
                    uint4 v = *reinterpret_cast<const uint4*>(p.res + oidx);
                    rw[0] = v.x; rw[1] = v.y; rw[2] = v.z; rw[3] = v.w;
                } else {
                    for (int j = 0; j < 16 && ocb + j < p.c_out; ++j)
                        rw[j >> 2] |= (uint32_t)p.res[oidx + j] << (8 * (j & 3));
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

        int32_t q[16];
#pragma unroll
        for (int j = 0; j < 16; ++j)
            q[j] = requant_one(a[j], mult[j], add ? res_code(rw, j, p.res_type) : 0, add, relu, m_res, p);

        if (p.y_type == T_INT8 || p.y_type == T_UINT8) {
            uint32_t ow[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                ow[j] = (uint32_t)(q[4 * j] & 0xFF) | ((uint32_t)(q[4 * j + 1] & 0xFF) << 8) |
                        ((uint32_t)(q[4 * j + 2] & 0xFF) << 16) | ((uint32_t)(q[4 * j + 3] & 0xFF) << 24);
            if (p.vec_store) {
                *reinterpret_cast<uint4*>(p.y + oidx) = make_uint4(ow[0], ow[1], ow[2], ow[3]);
            } else {
                for (int j = 0; j < 16 && ocb + j < p.c_out; ++j) p.y[oidx + j] = (uint8_t)(q[j] & 0xFF);
            }
        } else {
            uint32_t ow[2] = {0, 0};
#pragma unroll
            for (int j = 0; j < 16; ++j) ow[j >> 3] |= (uint32_t)(q[j] & 0xF) << (4 * (j & 7));
            if (p.vec_store) {
                *reinterpret_cast<uint2*>(p.y + (oidx >> 1)) = make_uint2(ow[0], ow[1]);
            } else {
                for (int j = 0; j < 8 && ocb + 2 * j < p.c_out; ++j)
                    p.y[(oidx >> 1) + j] = (uint8_t)((ow[j >> 2] >> (8 * (j & 3))) & 0xFF);
            }
        }
    }
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_shape(const ConvParams& p, int gather, bool is_1x1, hipStream_t stream) {
    ConvParams q = p;
    q.n_oc_tiles = (p.c_out + BM - 1) / BM;
    const int64_t n_px = (p.m + BN - 1) / BN;
    const int64_t grid = n_px * q.n_oc_tiles;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
    dim3 g((unsigned)grid), b(256);
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

}  // namespace

hipError_t launch_qconv(const ConvParams& p, int gather, bool is_1x1, hipStream_t stream) {
    if (p.c_out <= 64) return launch_shape<64, 256, 1, 4>(p, gather, is_1x1, stream);
    return launch_shape<128, 128, 2, 2>(p, gather, is_1x1, stream);
}

}  // namespace iqnn
