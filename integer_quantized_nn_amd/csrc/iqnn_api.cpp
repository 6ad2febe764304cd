// iqnn_api.cpp -- the extern "C" entry points of libiqnn: argument validation,
// layer prepacking (folded bias, multipliers, reordered weights) and kernel
// dispatch.  Declarations and full contracts are in include/iqnn.h.
#include <hip/hip_runtime.h>

#include <cfenv>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <limits>
#include <string>
#include <vector>

#include "iqnn.h"
#include "iqnn_internal.h"

#pragma clang fp contract(off)

namespace iqnn {

PackGeom pack_geom(int64_t c_out, int64_t k) {
    PackGeom g;
    g.ocp = (int32_t)((c_out + kOcPad - 1) / kOcPad * kOcPad);
    g.kp = (int32_t)((k + kKPad - 1) / kKPad * kKPad);
    g.w_off = (int64_t)g.ocp * 8 + 256;
    g.t_off = g.w_off + (int64_t)g.ocp * g.kp;
    g.bytes = g.t_off + (int64_t)g.ocp * g.kp;
    return g;
}

}  // namespace iqnn

using namespace iqnn;

namespace {

thread_local std::string g_err;

iqnn_status fail(iqnn_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

iqnn_status ok() {
    g_err.clear();
    return IQNN_OK;
}

bool code_range(int32_t t, int32_t* lo, int32_t* hi) {
    switch (t) {
    case T_INT8: *lo = -128; *hi = 127; return true;
    case T_UINT8: *lo = 0; *hi = 255; return true;
    case T_INT4: *lo = -8; *hi = 7; return true;
    case T_UINT4: *lo = 0; *hi = 15; return true;
    default: return false;
    }
}
bool is_code_type(int32_t t) { int32_t a, b; return code_range(t, &a, &b); }
bool is_sparse(int32_t w_type) { return w_type == T_INT8_2OF4; }
bool is_4bit(int32_t t) { return t == T_INT4 || t == T_UINT4; }
bool in_range(int32_t t, int32_t z) {
    int32_t lo, hi;
    return code_range(t, &lo, &hi) && z >= lo && z <= hi;
}
bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
bool scale_ok(float s) { return std::isfinite(s) && s > 0.0f; }
bool normal_ok(float s) { return std::isfinite(s) && s >= std::numeric_limits<float>::min(); }

// A conv or GEMM layer in one normalized form.
struct Layer {
    int64_t n, h, w, c, c_out, oh, ow, m, k;
    int32_t kh, kw, sh, sw, ph, pw;
    int32_t x_type, w_type, y_type, res_type, epi, z_in, z_out, z_res, z_w;
    bool int_rq;   // integer-only requantization (IQNN_EPI_INT_REQUANT)
    bool gemm;
};

// (M, N) of a positive binary32 multiplier x ~ M * 2^-N, M of kIntRqBits bits:
// N = clamp(bits - 1 - floor(log2 x), 0, 31), M = clamp(floor(x * 2^N), 0, 2^bits - 1),
// with floor(log2 x) the exact binary exponent (FQ-ViT article, LayerNorm code: get_MN).
constexpr int kIntRqBits = 8;
void int_multiplier(float x, int32_t* m, int32_t* n) {
    int e = 0;
    std::frexp((double)x, &e);   // x = f * 2^e, f in [0.5, 1): floor(log2 x) = e - 1
    const int32_t nn = std::min(std::max(kIntRqBits - 1 - (e - 1), 0), 31);
    const double scaled = std::floor(std::ldexp((double)x, nn));
    *n = nn;
    *m = (int32_t)std::min(std::max(scaled, 0.0), (double)((1 << kIntRqBits) - 1));
}

// Weights are held as q_W - s_w (s_w = 128 for UINT8, else 0) so every type fits
// int8; zw_red = s_w - Z_w is the coefficient of the per-pixel sum of the kernel's
// activation operands (MegEngine 4-bit article, 緩解精度下降: the red term).
int32_t weight_shift(const Layer& L) { return L.w_type == T_UINT8 ? 128 : 0; }
int32_t zw_red(const Layer& L) { return weight_shift(L) - L.z_w; }

iqnn_status check_layer(const Layer& L) {
    if (L.n <= 0 || L.h <= 0 || L.w <= 0 || L.c <= 0 || L.c_out <= 0)
        return fail(IQNN_ERR_INVALID_ARG, "sizes must be positive (n=%lld h=%lld w=%lld c_in=%lld c_out=%lld)",
                    (long long)L.n, (long long)L.h, (long long)L.w, (long long)L.c, (long long)L.c_out);
    if (L.kh <= 0 || L.kw <= 0 || L.sh <= 0 || L.sw <= 0 || L.ph < 0 || L.pw < 0)
        return fail(IQNN_ERR_INVALID_ARG, "kernel, stride must be positive and padding non-negative");
    if (L.h + 2 * (int64_t)L.ph < L.kh || L.w + 2 * (int64_t)L.pw < L.kw || L.oh <= 0 || L.ow <= 0)
        return fail(IQNN_ERR_INVALID_ARG, "kernel larger than the padded input");
    if (L.c_out > (1 << 24) || L.k > (1 << 24))
        return fail(IQNN_ERR_UNSUPPORTED, "C_out or K above 2^24");
    if (!is_code_type(L.x_type)) return fail(IQNN_ERR_INVALID_ARG, "activation type %d is not a code type", L.x_type);
    if (is_sparse(L.w_type)) {
        // 2:4 weights: symmetric int8 codes on the sparse streaming kernel
        if (L.z_w != 0) return fail(IQNN_ERR_INVALID_ARG, "2:4 weights are symmetric int8 codes (z_w must be 0)");
        const bool add = L.epi == E_ADD || L.epi == E_ADD_RELU;
        const bool is_1x1 = L.kh == 1 && L.kw == 1;
        if (is_4bit(L.x_type) || L.c % 64 != 0 || L.m >= ((int64_t)1 << 31) ||
            (!is_1x1 && (int64_t)L.kh * L.kw > 64) || L.int_rq ||
            (add && (is_4bit(L.res_type) || L.c_out % 16 != 0)))
            return fail(IQNN_ERR_UNSUPPORTED,
                        "2:4 weights need 8-bit activations, C_in %% 64 == 0, KH*KW <= 64, N*OH*OW < 2^31, the "
                        "binary32 requantization and an 8-bit residual with C_out %% 16 == 0");
    } else {
        if (!is_code_type(L.w_type)) return fail(IQNN_ERR_INVALID_ARG, "weight type %d is not a code type", L.w_type);
        if (!in_range(L.w_type, L.z_w)) return fail(IQNN_ERR_INVALID_ARG, "z_w %d outside the weight code range", L.z_w);
    }
    if (zw_red(L) != 0) {
        // the per-pixel term rides on the streaming kernel's 8-bit gather
        const bool add = L.epi == E_ADD || L.epi == E_ADD_RELU;
        const bool streamable = !is_4bit(L.x_type) && L.c % 64 == 0 && L.m < ((int64_t)1 << 31) &&
                                (int64_t)L.kh * L.kw <= 64 &&
                                (!add || (!is_4bit(L.res_type) && L.c_out % 16 == 0));
        if (!streamable)
            return fail(IQNN_ERR_UNSUPPORTED,
                        "weight zero point %d (w_type %d) needs 8-bit activations, C_in %% 64 == 0, KH*KW <= 64, "
                        "N*OH*OW < 2^31 and an 8-bit residual with C_out %% 16 == 0", L.z_w, L.w_type);
    }
    if (L.epi < E_NONE || L.epi > E_RAW) return fail(IQNN_ERR_INVALID_ARG, "unknown epilogue %d", L.epi);
    if (L.int_rq && L.epi != E_NONE && L.epi != E_RELU)
        return fail(IQNN_ERR_UNSUPPORTED, "integer-only requantization goes with NONE or RELU only");
    if (L.int_rq && zw_red(L) != 0)
        return fail(IQNN_ERR_UNSUPPORTED, "integer-only requantization takes weights without the Z_W term");
    if ((L.epi == E_RAW) != (L.y_type == T_INT32))
        return fail(IQNN_ERR_INVALID_ARG, "INT32 output goes with the RAW_INT32 epilogue and only with it");
    if (L.epi != E_RAW && !is_code_type(L.y_type))
        return fail(IQNN_ERR_INVALID_ARG, "output type %d is not a code type", L.y_type);
    const bool add = L.epi == E_ADD || L.epi == E_ADD_RELU;
    if (add && !is_code_type(L.res_type))
        return fail(IQNN_ERR_INVALID_ARG, "residual type %d is not a code type", L.res_type);
    if (!in_range(L.x_type, L.z_in)) return fail(IQNN_ERR_INVALID_ARG, "z_in %d outside the input code range", L.z_in);
    if (L.epi != E_RAW && !in_range(L.y_type, L.z_out))
        return fail(IQNN_ERR_INVALID_ARG, "z_out %d outside the output code range", L.z_out);
    if (add && !in_range(L.res_type, L.z_res))
        return fail(IQNN_ERR_INVALID_ARG, "z_res %d outside the residual code range", L.z_res);
    if (is_4bit(L.x_type) && L.c % 16 != 0)
        return fail(IQNN_ERR_UNSUPPORTED, "4-bit activations need C_in %% 16 == 0 (C_in=%lld)", (long long)L.c);
    if ((is_4bit(L.y_type) || (add && is_4bit(L.res_type))) && L.c_out % 2 != 0)
        return fail(IQNN_ERR_INVALID_ARG, "4-bit outputs / residuals need an even C_out");
    if (is_4bit(L.w_type) && L.c % 2 != 0)
        return fail(IQNN_ERR_INVALID_ARG, "4-bit weights need an even C_in (nibble pairs)");
    if (!is_4bit(L.x_type) && L.c % 16 != 0 && L.w > 0x7FFFFFFF)
        return fail(IQNN_ERR_UNSUPPORTED, "element-gather path limited to 2^31 columns");
    if (L.m > ((int64_t)1 << 40)) return fail(IQNN_ERR_UNSUPPORTED, "too many output pixels");
    return IQNN_OK;
}

iqnn_status conv_layer(const iqnn_conv_desc* d, Layer* L) {
    if (!d) return fail(IQNN_ERR_INVALID_ARG, "null descriptor");
    L->gemm = false;
    L->n = d->n; L->h = d->h; L->w = d->w; L->c = d->c_in; L->c_out = d->c_out;
    L->kh = d->kh; L->kw = d->kw; L->sh = d->stride_h; L->sw = d->stride_w; L->ph = d->pad_h; L->pw = d->pad_w;
    L->x_type = d->x_type; L->w_type = d->w_type; L->y_type = d->y_type; L->res_type = d->res_type;
    L->epi = d->epilogue & ~IQNN_EPI_INT_REQUANT; L->int_rq = (d->epilogue & IQNN_EPI_INT_REQUANT) != 0;
    L->z_in = d->z_in; L->z_out = d->z_out; L->z_res = d->z_res; L->z_w = d->z_w;
    L->oh = L->sh > 0 ? (L->h + 2 * (int64_t)L->ph - L->kh) / L->sh + 1 : 0;
    L->ow = L->sw > 0 ? (L->w + 2 * (int64_t)L->pw - L->kw) / L->sw + 1 : 0;
    L->m = L->n * L->oh * L->ow;
    L->k = (int64_t)L->kh * L->kw * L->c;
    return check_layer(*L);
}

iqnn_status gemm_layer(const iqnn_gemm_desc* d, Layer* L) {
    if (!d) return fail(IQNN_ERR_INVALID_ARG, "null descriptor");
    L->gemm = true;
    L->n = 1; L->h = 1; L->w = d->m; L->c = d->k; L->c_out = d->n;
    L->kh = L->kw = L->sh = L->sw = 1; L->ph = L->pw = 0;
    L->x_type = d->a_type; L->w_type = d->b_type; L->y_type = d->c_type; L->res_type = d->res_type;
    L->epi = d->epilogue & ~IQNN_EPI_INT_REQUANT; L->int_rq = (d->epilogue & IQNN_EPI_INT_REQUANT) != 0;
    L->z_in = d->z_a; L->z_out = d->z_out; L->z_res = d->z_res; L->z_w = d->z_b;
    L->oh = 1; L->ow = d->m; L->m = d->m; L->k = d->k;
    if (d->m <= 0 || d->n <= 0 || d->k <= 0) return fail(IQNN_ERR_INVALID_ARG, "GEMM sizes must be positive");
    return check_layer(*L);
}

// The kernel configuration of one forward call (iqnn_kernel_cfg; NULL: automatic).
iqnn_status read_cfg(const iqnn_kernel_cfg* cfg, int* tile, int* xcd_groups) {
    *tile = -1;
    *xcd_groups = 0;
    if (!cfg) return IQNN_OK;
    if (cfg->tile < -1 || cfg->tile > kMaxTile)
        return fail(IQNN_ERR_INVALID_ARG, "kernel configuration: tile %d outside -1..%d", cfg->tile, kMaxTile);
    const int g = cfg->xcd_groups;
    if (g != 0 && g != 1 && g != 2 && g != 4 && g != 8)
        return fail(IQNN_ERR_INVALID_ARG, "kernel configuration: xcd_groups %d is not 0, 1, 2, 4 or 8", g);
    *tile = cfg->tile;
    *xcd_groups = g;
    return IQNN_OK;
}

// The 4-channel gather of the pipelined kernel: 8-bit activations with exactly 4
// channels and no padding (the input carries its own border, see
// iqnn_quantize_pad).  The filter row is widened to KWP in {4, 8, 16} taps (zero
// weights), so a stage of 64 K elements is a whole number of filter rows; the
// widened window of the last output column must still lie inside the input row.
int32_t c4_kwp(const Layer& L) { return L.kw <= 4 ? 4 : (L.kw <= 8 ? 8 : 16); }
bool c4_path(const Layer& L) {
    if (L.int_rq) return false;   // integer requantization runs on the register-staged kernel
    if (is_4bit(L.x_type) || L.c != 4 || L.ph != 0 || L.pw != 0 || L.kw > 16) return false;
    if (L.n * L.h * L.w >= ((int64_t)1 << 31)) return false;   // pixel indices are int32
    return (L.ow - 1) * (int64_t)L.sw + c4_kwp(L) <= L.w;
}
// K of the packed weights and of the kernel's loop.
int64_t kdim(const Layer& L) { return c4_path(L) ? (int64_t)L.kh * c4_kwp(L) * 4 : L.k; }


// Staged K position of logical K index k.  4-bit activations are unpacked in
// 16-element segments as [0,2,4,6, 1,3,5,7, 8,10,12,14, 9,11,13,15] (low nibbles of
// four bytes, then their high nibbles); the weights are stored in the same order
// so both MFMA operands see one consistent K permutation.
// stream4: the streaming kernel's 4-bit order, where a lane's one 16-byte read per
// 64-element stage carries its half of both 32-element k-steps: inside every group of
// 64 the 16-element blocks (1, 2) trade places, so channel block 2h + kk is K block
// 2kk + h.
int64_t staged_k(int64_t k, bool act4, bool stream4 = false) {
    if (!act4) return k;
    static const int pos_of_elem[16] = {0, 4, 1, 5, 2, 6, 3, 7, 8, 12, 9, 13, 10, 14, 11, 15};
    int64_t blk = (k >> 4) & 3;
    if (stream4 && (blk == 1 || blk == 2)) blk ^= 3;
    return (k & ~(int64_t)63) | (blk << 4) | pos_of_elem[k & 15];
}

// 4-bit activations take the streaming kernel when every 64-channel group lies inside
// one filter tap and the residual, if any, is 4-bit in whole 16-byte chunks.  The
// packed layout depends on this choice, so prepack and forward both ask here.
bool b4_stream(const Layer& L) {
    if (L.int_rq) return false;   // integer requantization runs on the register-staged kernel
    if (!is_4bit(L.x_type) || L.c % 64 != 0 || L.kh * L.kw > 64) return false;
    if (L.m >= ((int64_t)1 << 31)) return false;
    const bool add = L.epi == E_ADD || L.epi == E_ADD_RELU;
    if (add && (!is_4bit(L.res_type) || L.c_out % 32 != 0)) return false;
    return true;
}

// 4-bit streaming layers with INT4 weights and more than 64 output channels keep their
// weights packed in the tile-order copy: per (64-row group, 64-K stage) a 2 KB block of
// 32-byte rows, each the stage's 64 codes two per byte in K order (low nibble first, the
// layout of a 4-bit activation row), the row's 16-byte halves swapped on rows with bit 3
// set (the kernel's LDS swizzle).  The kernel unpacks them on chip as 16 * w, so its
// accumulator bound is 16 times the int8 path's (checked at prepack).
bool w4_packed(const Layer& L) {
    return b4_stream(L) && L.w_type == T_INT4 && L.z_w == 0 && L.c_out > 64;
}

// One output channel of 2:4 weights in the sparse kernel's layout (PackGeom): the
// weights are stored as the LDS image of every (128-row channel tile, 64-K stage)
// block, 5120 bytes each: 128 rows of 32 bytes of kept codes, then 128 rows of 8 bytes
// of positions.  A row's kept codes are, for each group of four K positions, the two
// kept codes in K order (zeros where fewer than two are nonzero); its 16-byte half h
// (K [32h, 32h + 32) of the stage) sits at slot h ^ ((row >> 3) & 1) of the row (the
// kernel's conflict-free LDS swizzle).  The positions of half h are the 32-bit word h,
// group g of the half in bits 4g..4g+3.  More than two nonzero codes in a group is an
// error (the weights are not 2:4 sparse).
iqnn_status pack_sparse_row(const std::vector<int32_t>& row, const PackGeom& g, int32_t oc, int8_t* wp) {
    const int64_t prow = packed_row_of_channel(oc);
    const int64_t tile = prow / kSpRows, r = prow % kSpRows;
    const int64_t nst = g.kp / 64;
    const int64_t k = (int64_t)row.size();
    for (int64_t s = 0; s < nst; ++s) {
        int8_t* blk = wp + (tile * nst + s) * kSpBlock;
        for (int64_t h = 0; h < 2; ++h) {
            int8_t* vals = blk + r * 32 + ((h ^ ((r >> 3) & 1)) * 16);
            uint32_t word = 0;
            for (int64_t gi = 0; gi < 8; ++gi) {
                const int64_t k0 = s * 64 + h * 32 + gi * 4;
                int kept[2], n = 0;
                for (int j = 0; j < 4; ++j) {
                    const int32_t v = k0 + j < k ? row[(size_t)(k0 + j)] : 0;
                    if (v == 0) continue;
                    if (n == 2)
                        return fail(IQNN_ERR_INVALID_ARG,
                                    "2:4 weights: channel %d has more than two nonzero codes in K %lld..%lld", oc,
                                    (long long)k0, (long long)k0 + 3);
                    kept[n++] = j;
                }
                // fill with zero positions, keeping the two positions distinct and increasing
                for (int j = 0; n < 2 && j < 4; ++j)
                    if (!(n == 1 && kept[0] == j)) kept[n++] = j;
                if (kept[0] > kept[1]) std::swap(kept[0], kept[1]);
                for (int q = 0; q < 2; ++q) {
                    const int64_t kk = k0 + kept[q];
                    vals[2 * gi + q] = (int8_t)(kk < k ? row[(size_t)kk] : 0);
                    word |= (uint32_t)kept[q] << (4 * gi + 2 * q);
                }
            }
            std::memcpy(blk + kSpRows * 32 + r * 8 + h * 4, &word, 4);
        }
    }
    return IQNN_OK;
}

// 4-bit streaming layers with INT4 weights also carry a BF6 copy of their weights for
// the FP6 MFMA path (chosen with kTileFp6), after the standard layout: int32 bias[ocp]
// (the folded bias plus the activation shift -- 8 for UINT4, 0 for INT4 -- times the
// channel's weight sum, since the path contracts q - 8) and 4 KB blocks per (64-row
// group, 64-K stage), group-major: 64-byte rows (the kernel's LDS image) whose 8-byte
// unit u (0-5: the 24 bytes of K half u / 3, 32 six-bit codes in K order) sits at unit
// u ^ ((row >> 2) & 7).  The fp32 accumulation is exact while 64 * K < 2^24.
bool b4f6(const Layer& L) { return b4_stream(L) && L.w_type == T_INT4 && L.z_w == 0 && 64 * L.k < (1 << 24); }
int64_t f6_bias_off(const Layer& L) { return pack_geom(L.c_out, kdim(L)).bytes; }
int64_t f6_w_off(const Layer& L) {
    const PackGeom g = pack_geom(L.c_out, kdim(L));
    return g.bytes + (int64_t)g.ocp * 4;
}
int64_t packed_size(const Layer& L) {
    const PackGeom g = pack_geom(L.c_out, kdim(L));
    return g.bytes + (b4f6(L) ? (int64_t)g.ocp * 4 + (int64_t)g.ocp * g.kp : 0);
}

// BF6 (e3m2) code of an integer in [-8, 8] (every one of them is exact).
uint32_t bf6_host(int v) {
    static const uint32_t mag[9] = {0, 12, 16, 18, 20, 21, 22, 23, 24};
    return (v < 0 ? 32u : 0u) | mag[v < 0 ? -v : v];
}

// One channel's BF6 codes into the FP6 blocks (see b4f6).
void put_f6_row(const std::vector<int32_t>& row, int64_t k, int64_t prow, int64_t nst, uint8_t* blocks) {
    for (int64_t s = 0; s < nst; ++s) {
        uint8_t* rp = blocks + ((prow / 64) * nst + s) * 4096 + (prow % 64) * 64;
        for (int64_t h = 0; h < 2; ++h) {
            uint8_t bytes[24] = {0};
            for (int v = 0; v < 32; ++v) {
                const int64_t kk = s * 64 + h * 32 + v;
                const uint32_t code = bf6_host(kk < k ? row[(size_t)kk] : 0);
                for (int b = 0; b < 6; ++b)
                    if ((code >> b) & 1u) bytes[(6 * v + b) / 8] |= (uint8_t)(1u << ((6 * v + b) % 8));
            }
            for (int i = 0; i < 3; ++i)
                std::memcpy(rp + (((3 * h + i) ^ ((prow >> 2) & 7)) * 8), bytes + 8 * i, 8);
        }
    }
}

// Writes the packed layer (layout in PackGeom) into host memory `dst` of packed_size(L).
iqnn_status prepack_into(const Layer& L, const void* w_host, const float* bias_host, float s_in,
                         const float* s_w_host, int per_channel, float s_out, float s_res, uint8_t* dst) {
    const PackGeom g = pack_geom(L.c_out, kdim(L));
    const bool c4 = c4_path(L);
    const bool b4s = b4_stream(L);
    const int64_t kwp = c4_kwp(L);
    if (!scale_ok(s_in)) return fail(IQNN_ERR_INVALID_ARG, "input scale must be positive and finite");
    const bool raw = L.epi == E_RAW;
    const bool add = L.epi == E_ADD || L.epi == E_ADD_RELU;
    if (!raw && !scale_ok(s_out)) return fail(IQNN_ERR_INVALID_ARG, "output scale must be positive and finite");
    if (add && !scale_ok(s_res)) return fail(IQNN_ERR_INVALID_ARG, "residual scale must be positive and finite");
    if (std::fegetround() != FE_TONEAREST) return fail(IQNN_ERR_INVALID_ARG, "host rounding mode is not nearest-even");

    std::memset(dst, 0, (size_t)packed_size(L));
    const bool f6 = b4f6(L);
    const bool w4 = w4_packed(L);
    int32_t* bias_f6 = f6 ? reinterpret_cast<int32_t*>(dst + f6_bias_off(L)) : nullptr;
    uint8_t* blocks_f6 = f6 ? dst + f6_w_off(L) : nullptr;
    int32_t* bias = reinterpret_cast<int32_t*>(dst);
    float* mult = reinterpret_cast<float*>(dst + (size_t)g.ocp * 4);
    float* mres = reinterpret_cast<float*>(dst + (size_t)g.ocp * 8 + kHdrMres);
    // padding row: raw Z_in codes (two per byte for 4-bit activations)
    const int pad_code = is_4bit(L.x_type) ? ((L.z_in & 0xF) | ((L.z_in & 0xF) << 4)) : (L.z_in & 0xFF);
    std::memset(dst + (size_t)g.ocp * 8 + kHdrPad, pad_code, 64);
    int8_t* wp = reinterpret_cast<int8_t*>(dst + g.w_off);

    const bool act4 = is_4bit(L.x_type);
    const int64_t shift = L.x_type == T_UINT8 ? 128 : 0;   // kernel stages q - 128 for UINT8
    const int64_t mx = L.x_type == T_UINT4 ? 15 : (L.x_type == T_INT4 ? 8 : 128);
    const uint8_t* wb = static_cast<const uint8_t*>(w_host);
    std::vector<int32_t> row((size_t)L.k);
    std::vector<int32_t> wrows(w4 ? (size_t)(L.c_out * L.k) : 0);   // every channel's codes (packed copy)

    for (int64_t oc = 0; oc < L.c_out; ++oc) {
        int64_t sum = 0, abs_sum = 0;
        for (int64_t k = 0; k < L.k; ++k) {
            int64_t e = oc * L.k + k;
            int32_t v;
            if (L.w_type == T_INT8 || is_sparse(L.w_type)) {
                v = (int8_t)wb[e];
            } else if (L.w_type == T_UINT8) {
                v = (int32_t)wb[e] - 128;   // held as q_W - 128
            } else {
                uint8_t byte = wb[e >> 1];
                v = (e & 1) ? (byte >> 4) : (byte & 0xF);
                if (L.w_type == T_INT4 && v >= 8) v -= 16;
            }
            row[(size_t)k] = v;
            if (w4) wrows[(size_t)(oc * L.k + k)] = v;
            sum += v;
            abs_sum += v < 0 ? -v : v;
        }
        const float s_w = per_channel ? s_w_host[oc] : s_w_host[0];
        if (!scale_ok(s_w)) return fail(IQNN_ERR_INVALID_ARG, "weight scale of channel %lld is not positive finite", (long long)oc);
        const float sw_in = s_in * s_w;
        int64_t bias_q = 0;
        if (bias_host) {
            const float b = bias_host[oc];
            if (!std::isfinite(b)) return fail(IQNN_ERR_INVALID_ARG, "bias of channel %lld is not finite", (long long)oc);
            const float rb = std::nearbyint(b / sw_in);
            if (!(rb >= -2147483648.0f && rb <= 2147483520.0f))
                return fail(IQNN_ERR_OVERFLOW, "quantized bias of channel %lld leaves int32", (long long)oc);
            bias_q = (int64_t)rb;
        }
        const int64_t red = zw_red(L);   // nonzero only on the 8-bit streaming path (checked)
        const int64_t fold = bias_q + (shift - L.z_in) * sum + L.k * (shift - L.z_in) * red;
        if (fold < INT32_MIN || fold > INT32_MAX)
            return fail(IQNN_ERR_OVERFLOW, "folded bias of channel %lld leaves int32", (long long)oc);
        if (mx * abs_sum + (fold < 0 ? -fold : fold) + (red < 0 ? -red : red) * mx * L.k > INT32_MAX)
            return fail(IQNN_ERR_OVERFLOW, "accumulator of channel %lld may leave int32", (long long)oc);
        if (w4 && 16 * (mx * abs_sum + (fold < 0 ? -fold : fold)) > INT32_MAX)
            return fail(IQNN_ERR_OVERFLOW, "accumulator of channel %lld may leave int32 on the packed INT4 path "
                        "(16 times the bound)", (long long)oc);
        bias[oc] = (int32_t)fold;
        if (f6) {   // the FP6 path contracts (q - 8) for UINT4 activations
            const int64_t f = fold + (L.x_type == T_UINT4 ? 8 : 0) * sum;
            if (f < INT32_MIN || f > INT32_MAX)
                return fail(IQNN_ERR_OVERFLOW, "folded bias of channel %lld leaves int32", (long long)oc);
            bias_f6[oc] = (int32_t)f;   // physical channel order, like the folded bias
            put_f6_row(row, L.k, packed_row_of_channel((int32_t)oc), g.kp / 64, blocks_f6);
        }
        if (!raw) {
            const float m = sw_in / s_out;
            if (!normal_ok(m) || m > 1e20f)
                return fail(IQNN_ERR_INVALID_ARG, "requant multiplier of channel %lld is not a normal float in [FLT_MIN, 1e20]", (long long)oc);
            if (L.int_rq) {   // the slot holds M_c * 2^-N_c, exact in binary32 (8-bit M_c, N_c <= 31)
                int32_t mi, ni;
                int_multiplier(m, &mi, &ni);
                mult[oc] = std::ldexp((float)mi, -ni);
            } else {
                mult[oc] = m;
            }
        } else {
            mult[oc] = 1.0f;
        }
        if (is_sparse(L.w_type)) {
            iqnn_status st = pack_sparse_row(row, g, (int32_t)oc, wp);
            if (st != IQNN_OK) return st;
            continue;
        }
        int8_t* dst = wp + (int64_t)packed_row_of_channel((int32_t)oc) * g.kp;
        for (int64_t k = 0; k < L.k; ++k) {
            int64_t pos = staged_k(k, act4, b4s);
            if (c4) {   // (kh, kw, ci) -> (kh, kw in a row widened to kwp taps, ci)
                const int64_t kh = k / (L.kw * 4), kw = (k / 4) % L.kw, ci = k % 4;
                pos = (kh * kwp + kw) * 4 + ci;
            }
            dst[pos] = (int8_t)row[(size_t)k];
        }
    }
    if (add) {
        const float m = s_res / s_out;
        if (!normal_ok(m) || m > 1e20f)
            return fail(IQNN_ERR_INVALID_ARG, "residual multiplier is not a normal float in [FLT_MIN, 1e20]");
        mres[0] = m;
    }
    if (w4) {
        // packed INT4 tile-order copy (see w4_packed): block (row / 64, stage), 32 bytes
        // per row, half h at slot h ^ ((row >> 3) & 1)
        const int64_t nst = g.kp / 64;
        uint8_t* tp = dst + g.t_off;
        for (int64_t oc = 0; oc < L.c_out; ++oc) {
            const int64_t r = packed_row_of_channel((int32_t)oc);
            for (int64_t s = 0; s < nst; ++s) {
                uint8_t* rowp = tp + ((r / 64) * nst + s) * 2048 + (r % 64) * 32;
                for (int64_t i = 0; i < 64; ++i) {
                    const int64_t k = s * 64 + i;
                    const uint32_t code = k < L.k ? (uint32_t)wrows[(size_t)(oc * L.k + k)] & 0xFu : 0u;
                    const int64_t byte = i / 2, half = byte / 16;
                    const int64_t at = ((half ^ ((r >> 3) & 1)) * 16) + (byte % 16);
                    rowp[at] |= (uint8_t)(code << (4 * (i & 1)));
                }
            }
        }
    } else if (!is_sparse(L.w_type)) {
        // tile-order copy for the streaming kernel: block (row / 64, stage) holds, for
        // each of its 64 rows, the stage's four 16-byte K segments at slots q ^ swz(row)
        const int64_t nst = g.kp / 64;
        int8_t* tp = reinterpret_cast<int8_t*>(dst + g.t_off);
        for (int64_t r = 0; r < g.ocp; ++r) {
            const int64_t sw = (r >> 2) & 3;
            for (int64_t s = 0; s < nst; ++s) {
                int8_t* blk = tp + ((r / 64) * nst + s) * 4096 + (r % 64) * 64;
                for (int64_t q = 0; q < 4; ++q)
                    std::memcpy(blk + q * 16, wp + r * g.kp + s * 64 + (q ^ sw) * 16, 16);
            }
        }
    }
    return ok();
}

iqnn_status prepack_host(const Layer& L, const void* w_host, const float* bias_host, float s_in,
                         const float* s_w_host, int per_channel, float s_out, float s_res, void* packed_host,
                         size_t packed_bytes) {
    if (!w_host || !s_w_host || !packed_host) return fail(IQNN_ERR_INVALID_ARG, "null weight, scale or output pointer");
    const int64_t need = packed_size(L);
    if ((int64_t)packed_bytes < need)
        return fail(IQNN_ERR_INVALID_ARG, "packed buffer has %zu bytes, needs %lld", packed_bytes, (long long)need);
    return prepack_into(L, w_host, bias_host, s_in, s_w_host, per_channel, s_out, s_res,
                        static_cast<uint8_t*>(packed_host));
}

iqnn_status prepack_dev(const Layer& L, const void* w_host, const float* bias_host, float s_in,
                        const float* s_w_host, int per_channel, float s_out, float s_res, void* packed_dev,
                        size_t packed_bytes, hipStream_t stream) {
    if (!w_host || !s_w_host || !packed_dev) return fail(IQNN_ERR_INVALID_ARG, "null weight, scale or output pointer");
    const int64_t need = packed_size(L);
    if ((int64_t)packed_bytes < need)
        return fail(IQNN_ERR_INVALID_ARG, "packed buffer has %zu bytes, needs %lld", packed_bytes, (long long)need);
    if (!aligned(packed_dev, 256)) return fail(IQNN_ERR_ALIGNMENT, "packed buffer must be 256-byte aligned");
    std::vector<uint8_t> buf((size_t)need);
    iqnn_status s = prepack_into(L, w_host, bias_host, s_in, s_w_host, per_channel, s_out, s_res, buf.data());
    if (s != IQNN_OK) return s;
    hipError_t e = hipMemcpyAsync(packed_dev, buf.data(), buf.size(), hipMemcpyHostToDevice, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return fail(IQNN_ERR_HIP, "copy of the packed layer failed: %s", hipGetErrorString(e));
    return ok();
}

// Kernel parameters of a validated layer and its pointers.
void conv_params(const Layer& L, const void* x, const void* packed, const void* res, void* y, ConvParams& p,
                 bool f6 = false) {
    const bool add = L.epi == E_ADD || L.epi == E_ADD_RELU;
    const PackGeom g = pack_geom(L.c_out, kdim(L));
    const bool c4 = c4_path(L);
    std::memset(&p, 0, sizeof p);
    p.x = static_cast<const uint8_t*>(x);
    p.w = reinterpret_cast<const int8_t*>(static_cast<const uint8_t*>(packed) + g.w_off);
    p.w_tiled = reinterpret_cast<const int8_t*>(static_cast<const uint8_t*>(packed) + g.t_off);
    p.bias = static_cast<const int32_t*>(packed);
    p.mult = reinterpret_cast<const float*>(static_cast<const uint8_t*>(packed) + (size_t)g.ocp * 4);
    p.m_res = reinterpret_cast<const float*>(static_cast<const uint8_t*>(packed) + (size_t)g.ocp * 8 + kHdrMres);
    p.pad_row = static_cast<const uint8_t*>(packed) + (size_t)g.ocp * 8 + kHdrPad;
    // 2:4 weights: w_idx marks the sparse layout (the positions sit inside each block)
    p.w_idx = is_sparse(L.w_type) ? static_cast<const uint8_t*>(packed) + g.w_off + kSpRows * 32 : nullptr;
    p.res = add ? static_cast<const uint8_t*>(res) : nullptr;
    p.y = static_cast<uint8_t*>(y);
    p.m = L.m;
    p.h = (int32_t)L.h;
    p.w_in = (int32_t)(L.w > 0x7FFFFFFF ? 0x7FFFFFFF : L.w);
    p.c = (int32_t)L.c;
    p.oh = (int32_t)(L.oh > 0x7FFFFFFF ? 0x7FFFFFFF : L.oh);
    p.ow = (int32_t)(L.ow > 0x7FFFFFFF ? 0x7FFFFFFF : L.ow);
    p.kh = L.kh; p.kw = c4 ? c4_kwp(L) : L.kw; p.sh = L.sh; p.sw = L.sw; p.ph = L.ph; p.pw = L.pw;
    p.k = (int32_t)kdim(L);
    p.kp = g.kp;
    p.c_out = (int32_t)L.c_out;
    const uint32_t pad_byte = (L.x_type == T_UINT8) ? ((uint32_t)L.z_in ^ 0x80u) & 0xFF : (uint32_t)L.z_in & 0xFF;
    p.pad_word = pad_byte * 0x01010101u;
    p.x_xor = L.x_type == T_UINT8 ? 0x80808080u : 0u;
    p.x_signed4 = L.x_type == T_INT4;
    p.y_type = L.y_type;
    p.res_type = L.res_type;
    p.epi = L.epi;
    p.z_out = L.z_out;
    p.z_res = L.z_res;
    p.zw_red = zw_red(L);
    if (L.epi != E_RAW) {
        int32_t lo, hi;
        code_range(L.y_type, &lo, &hi);
        const bool relu = L.epi == E_RELU || L.epi == E_ADD_RELU;
        const int32_t low = relu ? std::max(lo, L.z_out) : lo;   // passive ReLU: clamp at Z_out
        const int32_t fix = L.int_rq ? 0 : (L.z_out & 1);        // odd part (two's complement)
        p.t_lo = (float)(low - L.z_out);
        p.t_hi = (float)(hi - L.z_out);
        p.q_lo = low - L.z_out;
        p.q_hi = hi - L.z_out;
        p.int_rq = L.int_rq ? 1 : 0;
        p.out_magic = 12582912.0f + (float)(L.z_out - fix);      // 1.5 * 2^23 + even part of Z_out
        // bytes hold code - fix; with no code 0 in [low, hi] none is 0xFF before the fix
        const bool packed_fix = fix && (L.y_type == T_UINT8 || L.y_type == T_INT8) && (low > 0 || hi < 0);
        p.out_fix = packed_fix ? 0u : (uint32_t)fix;
        p.out_fix4 = packed_fix ? 0x01010101u : 0u;
    }
    if (L.epi == E_ADD || L.epi == E_ADD_RELU) {
        const int32_t rshift = L.res_type == T_INT8 ? 128 : (L.res_type == T_INT4 ? 8 : 0);
        p.res_zf = (float)(L.z_res + rshift);
        p.res_xor = L.res_type == T_INT8 ? 0x80808080u : (L.res_type == T_INT4 ? 0x88888888u : 0u);
    }
    p.vec_store = L.c_out % 16 == 0;
    if (f6) {   // the layer's BF6 region (see b4f6)
        p.bias = reinterpret_cast<const int32_t*>(static_cast<const uint8_t*>(packed) + f6_bias_off(L));
        p.w_tiled = reinterpret_cast<const int8_t*>(static_cast<const uint8_t*>(packed) + f6_w_off(L));
        p.f6 = 1;
    }
}

iqnn_status forward(const Layer& L, const void* x, const void* packed, const void* res, void* y,
                    const iqnn_kernel_cfg* cfg, hipStream_t stream) {
    int tile, xcd_groups;
    if (iqnn_status st = read_cfg(cfg, &tile, &xcd_groups); st != IQNN_OK) return st;
    const bool add = L.epi == E_ADD || L.epi == E_ADD_RELU;
    if (!x || !packed || !y) return fail(IQNN_ERR_INVALID_ARG, "null input, packed or output pointer");
    if (add && !res) return fail(IQNN_ERR_INVALID_ARG, "ADD / ADD_RELU epilogue needs a residual");
    if (!aligned(x, 16) || !aligned(y, 16) || (add && !aligned(res, 16)))
        return fail(IQNN_ERR_ALIGNMENT, "activation, output and residual pointers must be 16-byte aligned");
    if (!aligned(packed, 256)) return fail(IQNN_ERR_ALIGNMENT, "packed buffer must be 256-byte aligned");
    const bool c4 = c4_path(L);
    ConvParams p;
    conv_params(L, x, packed, res, y, p, tile == kTileFp6 && b4f6(L));
    p.xcd_force = xcd_groups;
    p.w4 = w4_packed(L) && !p.f6;
    const int gather = is_4bit(L.x_type) ? (b4_stream(L) ? GATHER_B4S : GATHER_B4)
                                          : (L.c % 16 == 0 ? GATHER_B8 : (c4 ? GATHER_C4 : GATHER_B8_ELEM));
    const bool is_1x1 = gather != GATHER_B8_ELEM && gather != GATHER_C4 && L.kh == 1 && L.kw == 1 && L.sh == 1 && L.sw == 1 &&
                        L.ph == 0 && L.pw == 0;
    hipError_t e = launch_qconv(p, gather, is_1x1, stream, tile);
    if (e != hipSuccess) return fail(IQNN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

// Convolution followed by max pooling of its codes, fused (the image stem's shape
// class; see iqnn_qconv_maxpool_fwd).
iqnn_status forward_pool(const Layer& L, const void* x, const void* packed, void* y_pool, int32_t pool_k,
                         int32_t pool_stride, int32_t pool_pad, hipStream_t stream) {
    if (!x || !packed || !y_pool) return fail(IQNN_ERR_INVALID_ARG, "null input, packed or output pointer");
    if (!aligned(x, 16) || !aligned(y_pool, 16))
        return fail(IQNN_ERR_ALIGNMENT, "activation and output pointers must be 16-byte aligned");
    if (!aligned(packed, 256)) return fail(IQNN_ERR_ALIGNMENT, "packed buffer must be 256-byte aligned");
    if (pool_k != 3 || pool_stride != 2 || pool_pad != 1)
        return fail(IQNN_ERR_UNSUPPORTED, "fused pooling is 3x3, stride 2, padding 1 only");
    if (L.epi != E_NONE && L.epi != E_RELU)
        return fail(IQNN_ERR_UNSUPPORTED, "fused pooling takes Conv / Conv_Relu epilogues");
    if (!c4_path(L) || zw_red(L) != 0)
        return fail(IQNN_ERR_UNSUPPORTED, "fused pooling needs the 4-channel padding-free stem input");
    if (L.int_rq) return fail(IQNN_ERR_UNSUPPORTED, "fused pooling takes the binary32 requantization only");
    ConvParams p;
    conv_params(L, x, packed, nullptr, nullptr, p);
    if (!stem_pool_ok(p))
        return fail(IQNN_ERR_UNSUPPORTED,
                    "fused pooling needs a stride-2 stem with KH <= 8, 64 8-bit output channels, an even "
                    "input width, even OH and OW, OW <= 248, (KH+2)*W*4 <= 9200 and an input of N*H*W*4 "
                    "bytes divisible by 16");
    hipError_t e = launch_stem_pool(p, static_cast<uint8_t*>(y_pool), stream);
    if (e != hipSuccess) return fail(IQNN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

// Two 1x1 convs, the second reading the first's output (see iqnn_qconv_pair_fwd): one
// fused launch where the shapes allow, else the two calls one after the other.
iqnn_status forward_pair(const Layer& A, const Layer& Bl, const void* x, const void* packed_a, const void* res,
                         const void* packed_b, void* y_a, void* y_b, hipStream_t stream) {
    if (Bl.gemm || A.gemm || Bl.n != A.n || Bl.h != A.oh || Bl.w != A.ow || Bl.c != A.c_out ||
        Bl.x_type != A.y_type || Bl.z_in != A.z_out)
        return fail(IQNN_ERR_INVALID_ARG,
                    "the second conv's input (N, H, W, C_in, x_type, z_in) must be the first conv's output");
    // the checks of both calls before anything is launched
    const bool add = A.epi == E_ADD || A.epi == E_ADD_RELU;
    if (!x || !packed_a || !packed_b || !y_a || !y_b)
        return fail(IQNN_ERR_INVALID_ARG, "null input, packed or output pointer");
    if (add && !res) return fail(IQNN_ERR_INVALID_ARG, "ADD / ADD_RELU epilogue needs a residual");
    if (!aligned(x, 16) || !aligned(y_a, 16) || !aligned(y_b, 16) || (add && !aligned(res, 16)))
        return fail(IQNN_ERR_ALIGNMENT, "activation, output and residual pointers must be 16-byte aligned");
    if (!aligned(packed_a, 256) || !aligned(packed_b, 256))
        return fail(IQNN_ERR_ALIGNMENT, "packed buffers must be 256-byte aligned");
    {
        ConvParams pa, pb;
        conv_params(A, x, packed_a, res, y_a, pa);
        conv_params(Bl, y_a, packed_b, nullptr, y_b, pb);
        pa.w4 = w4_packed(A);
        pb.w4 = w4_packed(Bl);
        if (pair_ok(pa, pb)) {
            hipError_t e = launch_pair(pa, pb, stream);
            if (e != hipSuccess) return fail(IQNN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
            return ok();
        }
    }
    // every other pair: the two calls in order
    iqnn_status s = forward(A, x, packed_a, res, y_a, nullptr, stream);
    if (s != IQNN_OK) return s;
    return forward(Bl, y_a, packed_b, nullptr, y_b, nullptr, stream);
}

}  // namespace

extern "C" {

int iqnn_abi_version(void) { return IQNN_ABI_VERSION; }

const char* iqnn_status_str(iqnn_status s) {
    switch (s) {
    case IQNN_OK: return "IQNN_OK";
    case IQNN_ERR_INVALID_ARG: return "IQNN_ERR_INVALID_ARG";
    case IQNN_ERR_UNSUPPORTED: return "IQNN_ERR_UNSUPPORTED";
    case IQNN_ERR_ALIGNMENT: return "IQNN_ERR_ALIGNMENT";
    case IQNN_ERR_OVERFLOW: return "IQNN_ERR_OVERFLOW";
    case IQNN_ERR_HIP: return "IQNN_ERR_HIP";
    }
    return "IQNN_ERR_UNKNOWN";
}

const char* iqnn_last_error(void) { return g_err.c_str(); }

iqnn_status iqnn_choose_qparams(float minv, float maxv, int32_t qtype, int symmetric, float* scale,
                                int32_t* zp) {
    int32_t lo, hi;
    if (!code_range(qtype, &lo, &hi)) return fail(IQNN_ERR_INVALID_ARG, "choose_qparams: type %d is not a code type", qtype);
    if (!scale || !zp) return fail(IQNN_ERR_INVALID_ARG, "choose_qparams: null output");
    if (!std::isfinite(minv) || !std::isfinite(maxv) || minv > maxv)
        return fail(IQNN_ERR_INVALID_ARG, "choose_qparams: range [%g, %g] is not a finite interval", minv, maxv);
    if (symmetric && lo >= 0) return fail(IQNN_ERR_INVALID_ARG, "choose_qparams: symmetric parameters need a signed type");
    const float mn = minv < 0.0f ? minv : 0.0f, mx = maxv > 0.0f ? maxv : 0.0f;
    float s;
    if (symmetric) {
        s = std::max(std::fabs(minv), std::fabs(maxv)) / (float)hi;
    } else {
        const float width = mx - mn;
        if (!std::isfinite(width)) return fail(IQNN_ERR_OVERFLOW, "choose_qparams: range width overflows binary32");
        s = width / (float)(hi - lo);
    }
    if (!(s >= std::numeric_limits<float>::min())) s = 1.0f;
    int32_t z = 0;
    if (!symmetric) {
        const int64_t t = (int64_t)std::nearbyint(mn / s);
        z = (int32_t)std::min<int64_t>(std::max<int64_t>(lo - t, lo), hi);
    }
    *scale = s;
    *zp = z;
    return ok();
}

iqnn_status iqnn_quantize(const float* x_dev, void* q_dev, int64_t outer, int64_t ch, int64_t inner,
                          const float* scale_dev, const int32_t* zp_dev, int per_channel, int32_t qtype,
                          void* stream) {
    int32_t lo, hi;
    if (!code_range(qtype, &lo, &hi)) return fail(IQNN_ERR_INVALID_ARG, "quantize: type %d is not a code type", qtype);
    if (outer < 0 || ch <= 0 || inner <= 0) return fail(IQNN_ERR_INVALID_ARG, "quantize: bad view sizes");
    const int64_t total = outer * ch * inner;
    if (total > 0 && (!x_dev || !q_dev || !scale_dev || !zp_dev))
        return fail(IQNN_ERR_INVALID_ARG, "quantize: null pointer");
    if (is_4bit(qtype) && total % 2) return fail(IQNN_ERR_INVALID_ARG, "quantize: 4-bit output needs an even element count");
    if (!aligned(x_dev, 16) || !aligned(q_dev, is_4bit(qtype) ? 8 : 16))
        return fail(IQNN_ERR_ALIGNMENT, "quantize: misaligned pointer");
    QuantParams p{x_dev, static_cast<uint8_t*>(q_dev), scale_dev, zp_dev, total, ch, inner,
                  per_channel ? 1 : 0, qtype, lo, hi};
    hipError_t e = launch_quantize(p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(IQNN_ERR_HIP, "quantize launch failed: %s", hipGetErrorString(e));
    return ok();
}

iqnn_status iqnn_dequantize(const void* q_dev, float* x_dev, int64_t outer, int64_t ch, int64_t inner,
                            const float* scale_dev, const int32_t* zp_dev, int per_channel, int32_t qtype,
                            void* stream) {
    if (!is_code_type(qtype)) return fail(IQNN_ERR_INVALID_ARG, "dequantize: type %d is not a code type", qtype);
    if (outer < 0 || ch <= 0 || inner <= 0) return fail(IQNN_ERR_INVALID_ARG, "dequantize: bad view sizes");
    const int64_t total = outer * ch * inner;
    if (total > 0 && (!x_dev || !q_dev || !scale_dev || !zp_dev))
        return fail(IQNN_ERR_INVALID_ARG, "dequantize: null pointer");
    if (is_4bit(qtype) && total % 2) return fail(IQNN_ERR_INVALID_ARG, "dequantize: 4-bit input needs an even element count");
    if (!aligned(x_dev, 16) || !aligned(q_dev, is_4bit(qtype) ? 8 : 16))
        return fail(IQNN_ERR_ALIGNMENT, "dequantize: misaligned pointer");
    DequantParams p{static_cast<const uint8_t*>(q_dev), x_dev, scale_dev, zp_dev, total, ch, inner,
                    per_channel ? 1 : 0, qtype};
    hipError_t e = launch_dequantize(p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(IQNN_ERR_HIP, "dequantize launch failed: %s", hipGetErrorString(e));
    return ok();
}

iqnn_status iqnn_quantize_pad(const float* x_dev, void* q_dev, int32_t n, int32_t h, int32_t w, int32_t c,
                              int32_t pad, int32_t c_pad, const float* scale_dev, const int32_t* zp_dev,
                              int per_channel, int32_t qtype, void* stream) {
    int32_t lo, hi;
    if (qtype != T_INT8 && qtype != T_UINT8) return fail(IQNN_ERR_UNSUPPORTED, "quantize_pad: 8-bit codes only");
    code_range(qtype, &lo, &hi);
    if (n < 0 || h <= 0 || w <= 0 || c <= 0 || pad < 0 || c_pad < c)
        return fail(IQNN_ERR_INVALID_ARG, "quantize_pad: bad sizes (need c_pad >= c, pad >= 0)");
    if ((int64_t)n * (h + 2 * pad) * (w + 2 * pad) >= ((int64_t)1 << 31) ||
        (int64_t)(h + 2 * pad) * (w + 2 * pad) * c_pad > ((int64_t)1 << 40))
        return fail(IQNN_ERR_UNSUPPORTED, "quantize_pad: N*(H+2pad)*(W+2pad) must be below 2^31");
    if (n > 0 && (!x_dev || !q_dev || !scale_dev || !zp_dev)) return fail(IQNN_ERR_INVALID_ARG, "quantize_pad: null pointer");
    if (!aligned(x_dev, 4) || !aligned(q_dev, 4)) return fail(IQNN_ERR_ALIGNMENT, "quantize_pad: misaligned pointer");
    QuantPadParams p{x_dev, static_cast<uint8_t*>(q_dev), scale_dev, zp_dev, n, h, w, c, pad, c_pad,
                     per_channel ? 1 : 0, lo, hi};
    hipError_t e = launch_quantize_pad(p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(IQNN_ERR_HIP, "quantize_pad launch failed: %s", hipGetErrorString(e));
    return ok();
}

size_t iqnn_qconv_packed_size(const iqnn_conv_desc* desc) {
    Layer L;
    if (conv_layer(desc, &L) != IQNN_OK) return 0;
    ok();
    return (size_t)packed_size(L);
}

iqnn_status iqnn_qconv_prepack(const iqnn_conv_desc* desc, const void* w_host, const float* bias_host, float s_in,
                               const float* s_w_host, int per_channel, float s_out, float s_res, void* packed_dev,
                               size_t packed_bytes, void* stream) {
    Layer L;
    iqnn_status s = conv_layer(desc, &L);
    if (s != IQNN_OK) return s;
    return prepack_dev(L, w_host, bias_host, s_in, s_w_host, per_channel, s_out, s_res, packed_dev, packed_bytes,
                       static_cast<hipStream_t>(stream));
}

iqnn_status iqnn_qconv_prepack_host(const iqnn_conv_desc* desc, const void* w_host, const float* bias_host,
                                    float s_in, const float* s_w_host, int per_channel, float s_out, float s_res,
                                    void* packed_host, size_t packed_bytes) {
    Layer L;
    iqnn_status s = conv_layer(desc, &L);
    if (s != IQNN_OK) return s;
    return prepack_host(L, w_host, bias_host, s_in, s_w_host, per_channel, s_out, s_res, packed_host, packed_bytes);
}

iqnn_status iqnn_qconv_fwd(const iqnn_conv_desc* desc, const void* x_dev, const void* packed_dev,
                           const void* res_dev, void* y_dev, void* stream) {
    return iqnn_qconv_fwd_cfg(desc, x_dev, packed_dev, res_dev, y_dev, nullptr, stream);
}

iqnn_status iqnn_qconv_fwd_cfg(const iqnn_conv_desc* desc, const void* x_dev, const void* packed_dev,
                               const void* res_dev, void* y_dev, const iqnn_kernel_cfg* cfg, void* stream) {
    Layer L;
    iqnn_status s = conv_layer(desc, &L);
    if (s != IQNN_OK) return s;
    return forward(L, x_dev, packed_dev, res_dev, y_dev, cfg, static_cast<hipStream_t>(stream));
}

iqnn_status iqnn_qconv_maxpool_fwd(const iqnn_conv_desc* desc, const void* x_dev, const void* packed_dev,
                                   void* y_dev, int32_t pool_k, int32_t pool_stride, int32_t pool_pad,
                                   void* stream) {
    Layer L;
    iqnn_status s = conv_layer(desc, &L);
    if (s != IQNN_OK) return s;
    return forward_pool(L, x_dev, packed_dev, y_dev, pool_k, pool_stride, pool_pad,
                        static_cast<hipStream_t>(stream));
}

iqnn_status iqnn_qconv_pair_fwd(const iqnn_conv_desc* desc_a, const iqnn_conv_desc* desc_b, const void* x_dev,
                                const void* packed_a_dev, const void* res_dev, const void* packed_b_dev,
                                void* y_a_dev, void* y_b_dev, void* stream) {
    Layer A, Bl;
    iqnn_status s = conv_layer(desc_a, &A);
    if (s != IQNN_OK) return s;
    s = conv_layer(desc_b, &Bl);
    if (s != IQNN_OK) return s;
    return forward_pair(A, Bl, x_dev, packed_a_dev, res_dev, packed_b_dev, y_a_dev, y_b_dev,
                        static_cast<hipStream_t>(stream));
}

size_t iqnn_qgemm_packed_size(const iqnn_gemm_desc* desc) {
    Layer L;
    if (gemm_layer(desc, &L) != IQNN_OK) return 0;
    ok();
    return (size_t)packed_size(L);
}

iqnn_status iqnn_qgemm_prepack(const iqnn_gemm_desc* desc, const void* b_host, const float* bias_host, float s_a,
                               const float* s_b_host, int per_channel, float s_out, float s_res, void* packed_dev,
                               size_t packed_bytes, void* stream) {
    Layer L;
    iqnn_status s = gemm_layer(desc, &L);
    if (s != IQNN_OK) return s;
    return prepack_dev(L, b_host, bias_host, s_a, s_b_host, per_channel, s_out, s_res, packed_dev, packed_bytes,
                       static_cast<hipStream_t>(stream));
}

iqnn_status iqnn_qgemm_prepack_host(const iqnn_gemm_desc* desc, const void* b_host, const float* bias_host,
                                    float s_a, const float* s_b_host, int per_channel, float s_out, float s_res,
                                    void* packed_host, size_t packed_bytes) {
    Layer L;
    iqnn_status s = gemm_layer(desc, &L);
    if (s != IQNN_OK) return s;
    return prepack_host(L, b_host, bias_host, s_a, s_b_host, per_channel, s_out, s_res, packed_host, packed_bytes);
}

iqnn_status iqnn_qgemm_fwd(const iqnn_gemm_desc* desc, const void* a_dev, const void* packed_dev,
                           const void* res_dev, void* c_dev, void* stream) {
    return iqnn_qgemm_fwd_cfg(desc, a_dev, packed_dev, res_dev, c_dev, nullptr, stream);
}

iqnn_status iqnn_qgemm_fwd_cfg(const iqnn_gemm_desc* desc, const void* a_dev, const void* packed_dev,
                               const void* res_dev, void* c_dev, const iqnn_kernel_cfg* cfg, void* stream) {
    Layer L;
    iqnn_status s = gemm_layer(desc, &L);
    if (s != IQNN_OK) return s;
    return forward(L, a_dev, packed_dev, res_dev, c_dev, cfg, static_cast<hipStream_t>(stream));
}

iqnn_status iqnn_probe_empty(void* stream) {
    hipError_t e = launch_probe_empty(static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(IQNN_ERR_HIP, "probe launch failed: %s", hipGetErrorString(e));
    return ok();
}

iqnn_status iqnn_probe_mfma_rate(int32_t iters, int32_t blocks, int32_t* sink_dev, void* stream) {
    if (iters <= 0 || blocks <= 0 || !sink_dev)
        return fail(IQNN_ERR_INVALID_ARG, "probe: iters and blocks must be positive and sink_dev non-null");
    if (!aligned(sink_dev, 4)) return fail(IQNN_ERR_ALIGNMENT, "probe: sink_dev must be 4-byte aligned");
    hipError_t e = launch_probe_mfma_rate(iters, blocks, sink_dev, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(IQNN_ERR_HIP, "probe launch failed: %s", hipGetErrorString(e));
    return ok();
}

iqnn_status iqnn_maxpool2d(const void* x_dev, void* y_dev, int32_t n, int32_t h, int32_t w, int32_t c, int32_t k,
                           int32_t stride, int32_t pad, int32_t dtype, void* stream) {
    if (dtype != T_INT8 && dtype != T_UINT8) return fail(IQNN_ERR_UNSUPPORTED, "maxpool: 8-bit codes only");
    if (n <= 0 || h <= 0 || w <= 0 || c <= 0 || k <= 0 || stride <= 0 || pad < 0)
        return fail(IQNN_ERR_INVALID_ARG, "maxpool: sizes must be positive");
    if (2 * pad > k - 1) return fail(IQNN_ERR_INVALID_ARG, "maxpool: padding must satisfy 2*pad <= k-1");
    if (c % 16 != 0) return fail(IQNN_ERR_UNSUPPORTED, "maxpool: C %% 16 != 0");
    if (h + 2 * pad < k || w + 2 * pad < k) return fail(IQNN_ERR_INVALID_ARG, "maxpool: window larger than input");
    {
        const int64_t ohp = (h + 2 * pad - k) / stride + 1, owp = (w + 2 * pad - k) / stride + 1;
        if ((int64_t)n * ohp * owp * (c / 16) >= ((int64_t)1 << 31))
            return fail(IQNN_ERR_UNSUPPORTED, "maxpool: N*OH*OW*C/16 must be below 2^31");
    }
    if (!x_dev || !y_dev) return fail(IQNN_ERR_INVALID_ARG, "maxpool: null pointer");
    if (!aligned(x_dev, 16) || !aligned(y_dev, 16)) return fail(IQNN_ERR_ALIGNMENT, "maxpool: misaligned pointer");
    PoolParams p{static_cast<const uint8_t*>(x_dev), static_cast<uint8_t*>(y_dev), n, h, w, c, k, stride, pad,
                 (h + 2 * pad - k) / stride + 1, (w + 2 * pad - k) / stride + 1, dtype == T_INT8};
    hipError_t e = launch_maxpool(p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(IQNN_ERR_HIP, "maxpool launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // extern "C"
