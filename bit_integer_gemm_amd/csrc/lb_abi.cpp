// lb_abi.cpp -- the extern "C" boundary declared in include/lb_gemm.h:
// argument checks, variant selection and launch on the caller's stream.
#include "lb_gemm.h"

#include <hip/hip_runtime.h>

#include <cstdlib>
#include <cstring>

#include "lb_internal.hpp"

#ifndef LB_SOURCE_SHA
#error "LB_SOURCE_SHA (hash of the source files) is set by the build"
#endif

namespace {

// The build stamps the hash of the source text into the library; the marker
// also lets a tool read it from the file without loading it.
const char kBuildMark[] = "lb-source-sha:" LB_SOURCE_SHA;

int check_common(const void *a, const void *b, const void *c, int64_t M, int64_t N, int64_t K,
                 int64_t align, int64_t kmax, int variant)
{
    if (!a || !b || !c) return LB_ERR_NULL;
    if (M <= 0 || N <= 0 || K <= 0) return LB_ERR_SHAPE;
    if (M > 0x7FFFFFFF || N > 0x7FFFFFFF) return LB_ERR_SHAPE;
    if (K % align != 0) return LB_ERR_ALIGN;
    if (variant < LB_AUTO || variant >= LB_NUM_VARIANTS) return LB_ERR_VARIANT;
    if (K > kmax) return LB_ERR_OVERFLOW;
    return LB_OK;
}

// LB_AUTO_VARIANT=v (0..8) in the environment replaces the selector's choice
// for LB_AUTO; the automatic path's splits still apply.  -1 when unset or not
// a variant index.
int auto_override()
{
    const char *e = std::getenv("LB_AUTO_VARIANT");
    if (!e || e[0] < '0' || e[0] > '8' || e[1] != '\0') return -1;
    return e[0] - '0';
}

int resolve(int dtype, int variant, int64_t M, int64_t N, int64_t K, int cu)
{
    if (variant != LB_AUTO) return variant;
    const int forced = auto_override();
    if (forced >= 0) return forced;
    int best = LB_DEFAULT_VARIANT;
    // cu_count 0: ask the current device; any failure keeps the default.
    if (lb::select_from_table(dtype, M, N, K, cu, &best, nullptr) != LB_OK) return LB_DEFAULT_VARIANT;
    return best;
}

int finish(hipError_t e) { return e == hipSuccess ? LB_OK : LB_ERR_HIP; }

// Wave quantisation.  The large tiles (variants 6-8) hold one workgroup per
// CU, so a grid of T tiles runs in ceil(T / CUs) rounds, and a last round at
// most half full leaves most CUs idle for a whole tile time (8192 x 11008 has
// 32 x 43 = 1376 tiles: 5 full rounds on 256 CUs and one of 96).  An automatic
// choice then runs the product as two launches on the stream: the widest band
// of leading tile columns (else tile rows) that fills whole rounds, and the
// rest as a product of its own with the variant chosen for that shape
// (measured: 1.20x at 4096 x 4864 x 4096, 1.31x at 4096 x 4608 x 8192).
struct Part {
    int64_t m0, m, n0, n;
    int variant;
};

int plan_parts(int dtype, int variant, int64_t M, int64_t N, int64_t K, int cu, Part *parts)
{
    parts[0] = {0, M, 0, N, variant};
    if (variant < 6 || cu <= 0) return 1;
    const int64_t tile = 256;
    const int64_t tm = (M + tile - 1) / tile, tn = (N + tile - 1) / tile, T = tm * tn;
    if (T <= cu || T % cu == 0 || 2 * (T % cu) > cu) return 1;
    int64_t c = tn - 1;
    while (c > 0 && (tm * c) % cu != 0) --c;
    if (c > 0) {
        const int64_t n1 = c * tile;
        parts[0] = {0, M, 0, n1, variant};
        parts[1] = {0, M, n1, N - n1, resolve(dtype, LB_AUTO, M, N - n1, K, cu)};
        return 2;
    }
    int64_t r = tm - 1;
    while (r > 0 && (r * tn) % cu != 0) --r;
    if (r > 0) {
        const int64_t m1 = r * tile;
        parts[0] = {0, m1, 0, N, variant};
        parts[1] = {m1, M - m1, 0, N, resolve(dtype, LB_AUTO, M - m1, N, K, cu)};
        return 2;
    }
    return 1;
}

// One partial round of the four-wave tile.  When an automatic choice for the
// int8 GEMM or the linear layer is the four-wave 256x256 tile (variant 6) and
// its grid has fewer tiles than the chip has CUs, the product runs on 256x192
// tiles instead (else 192x256, whichever grid is smaller) if that grid still
// fits in one round: every CU then does a quarter less work.  The int4 and
// 1-bit (FP4 route) GEMMs take the 256x192 tile the same way (their plane
// schedules exist for eight and six fragment columns, not for six rows).
// Measured on
// MI355X, identical results: 8192 x 1376 x 4096 (linear) 47.5 against 53.6
// us, 1024 x 11008 x 4096 (linear) 46.3 against 54.0 us, int8 4096 x 3072 x
// 4096 48.4 against 54.2 us, 3072 x 4096 x 4096 (192x256) 48.2 against 53.3 us.
// The narrow tile (W4_256x192 or W4_192x256) a product of this kind would take
// on one partial round, and its tile count; 0 if none applies.
int narrow_tile_of(int kind, int64_t M, int64_t N, int cu, int64_t *count)
{
    const bool s4 = kind == lb::KIND_S4 || kind == lb::KIND_B1F4;   // 256x192 only
    if ((kind != lb::KIND_S8 && kind != lb::KIND_LINEAR && !s4) || cu <= 0) return 0;
    auto tiles = [&](int64_t bm, int64_t bn) { return ((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
    if (tiles(256, 256) >= cu) return 0;
    const int64_t wide = tiles(256, 192), tall = tiles(192, 256);
    if (wide <= cu && (s4 || tall > cu || wide <= tall)) { *count = wide; return lb::W4_256x192; }
    if (tall <= cu && !s4) { *count = tall; return lb::W4_192x256; }
    return 0;
}

int narrow_w4_tile(int kind, int variant, int64_t M, int64_t N, int cu)
{
    int64_t count = 0;
    const int t = variant == 6 ? narrow_tile_of(kind, M, N, cu, &count) : 0;
    return t ? t : variant;
}

// A nearly full round of narrow tiles beats the selector's choice.  The
// selection table and network know the nine variants only.  Measured on MI355X
// over partial-round shapes (M x N from 1536 x 8192 to 5120 x 2304, int4 K 2048-
// 8192, 1-bit K 8192-32768 bits): where the narrow grid had at least 7/8 as many
// tiles as CUs, variant 6 on it was 1.12-1.16x faster (int4) and 1.11-1.22x
// (1-bit) than the medium tile the selector chose, on every shape; with 176 or
// fewer tiles the selector's choice was faster (1.01-1.32x).  The int8 selector
// already chose variant 6 on every shape above that fill.  An automatic choice
// (not one fixed by LB_AUTO_VARIANT) is therefore replaced by variant 6 there.
int prefer_full_narrow_round(int kind, int variant, int64_t M, int64_t N, int cu)
{
    if (variant == 6 || auto_override() >= 0 || cu <= 0) return variant;
    int64_t count = 0;
    if (narrow_tile_of(kind, M, N, cu, &count) && 8 * count >= 7 * (int64_t)cu) return 6;
    return variant;
}

// Launch a product, or for an automatic choice its parts.  kb is the bytes per
// row of A and B (B's rows are the output's columns); out_elem is the bytes of
// one output element.
// Split K.  A product whose tiles fill at most a quarter of the CUs (small
// M x N) leaves the chip mostly idle however long K is.  An automatic choice
// for an integer GEMM may then cut K into S bands of whole stages, zero C and
// run all bands in one grid, each adding its exact int32 partial sums into C
// with atomic adds; integer addition makes the result independent of their
// order.  S comes from a cost model fitted to measurements on MI355X: a
// one-round product takes about alpha ns per element of K (2.5 int8, 2.3 int4,
// 0.83 1-bit on the FP4 route, 1.25 on the int8 route); S bands take
// alpha K / S, plus ~3 us for the zeroing launch, plus ~15 ps per atomic add
// (M N S of them).  The S (2..16, at most
// CUs / tiles and whole 128-byte stages) with the lowest estimate is used when
// that estimate beats alpha K by 1.3x (measured: int8 64 x 64 x 8192 2.9x
// faster, 1-bit 64 x 64 x 32768 4.9x; the model declines 64 x 4096 x 4096 and
// 1-bit 4096 x 64 x 8192, where bands lost 9% and 47%).  Returns S (1: no
// split) and the band length in bytes.
int plan_ksplit(int kind, int variant, int64_t M, int64_t N, int64_t kb, int cu, int64_t *band)
{
    *band = kb;
    if (kind == lb::KIND_LINEAR || cu <= 0) return 1;  // the dequantisation needs the whole sum
    int bm = 0, bn = 0, bk = 0, st = 0;
    if (lb::mfma_variant_info(kind, variant, &bm, &bn, &bk, &st) != 0) return 1;
    const int64_t tiles = ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
    if (4 * tiles > cu) return 1;
    const int per_byte = kind == lb::KIND_S8 ? 1 : kind == lb::KIND_S4 ? 2 : 8;
    const double alpha = kind == lb::KIND_S8    ? 2.5
                         : kind == lb::KIND_S4  ? 2.3
                         : kind == lb::KIND_B1F4 ? 0.83
                                                 : 1.25;
    const double t0 = alpha * (double)kb * per_byte;
    const int64_t step = 128;  // a multiple of every variant's stage depth
    int64_t smax = cu / tiles;
    if (smax > 16) smax = 16;
    if (smax > kb / step) smax = kb / step;
    int best = 1;
    double best_t = t0;
    for (int64_t S = 2; S <= smax; ++S) {
        const double t = t0 / (double)S + 3000.0 + 0.015 * (double)M * (double)N * (double)S;
        if (t < best_t) { best_t = t; best = (int)S; }
    }
    if (best < 2 || best_t * 1.3 > t0) return 1;
    const int64_t len = ((kb + best - 1) / best + step - 1) / step * step;
    const int64_t bands = (kb + len - 1) / len;
    if (bands < 2) return 1;
    *band = len;
    return (int)bands;
}

// The 1-bit GEMM's matrix instruction: FP4 (four bit planes per 64-byte
// block, fp32 sums; one instruction covers 128 K bits) by default, or int8
// (eight weighted planes, int32 sums; 64 K bits per instruction).  Measured
// on MI355X, every variant, bit-identical results: FP4 1.27-1.59x faster
// (4096 x 4096 x 8192 bits 51.0 against 79.8 us, 8192^3 198.9 against 312.6
// us).  LB_B1_ROUTE=int8 in the environment selects the int8 route (for A/B
// measurement and its parity tests).
int b1_kind()
{
    const char *e = std::getenv("LB_B1_ROUTE");
    if (e && std::strcmp(e, "int8") == 0) return lb::KIND_B1;
    return lb::KIND_B1F4;
}

// 1-bit K limit of one pass.  The int8 route accumulates 64 per matching bit
// pair in int32, so one pass covers at most 33,554,304 bits (4,194,288 bytes
// per row); the FP4 route accumulates 1.0 per pair in fp32, exact up to 2^24
// (2,097,152 bytes).  A longer K runs as bands of whole 128-byte stages, each
// within the pass limit, that add their exact counts into C after a zero fill;
// this applies to every variant, not only to an automatic choice.
int64_t b1_pass_bytes(int kind) { return kind == lb::KIND_B1F4 ? 2097152 : 4194288; }

int64_t b1_band_bytes(int kind, int64_t kb)
{
    const int64_t pass = b1_pass_bytes(kind), bmax = pass / 128 * 128;
    if (kb <= pass) return kb;
    const int64_t bands = (kb + bmax - 1) / bmax;
    return ((kb + bands - 1) / bands + 127) / 128 * 128;
}

// The launches of one call: one or two parts of the output, the K band of a
// single part (kb: no bands), and whether C is zeroed first (K bands).
struct Plan {
    Part parts[2];
    int np;
    int64_t band;
    bool zero;
};

// cu: the CU count to plan for; <= 0 asks the current device (when the plan
// needs it), and a failed query plans as with no CU information (no splits,
// bands or narrow tiles; the selection falls back to the default variant).
Plan make_plan(int kind, int dtype, int variant, int64_t M, int64_t N, int64_t K, int64_t kb, int cu)
{
    Plan p{{{0, M, 0, N, variant}, {0, 0, 0, 0, 0}}, 1, kb, false};
    const bool b1 = kind == lb::KIND_B1 || kind == lb::KIND_B1F4;
    if (variant == LB_AUTO && cu <= 0 && lb::device_cu_count(&cu) != LB_OK) cu = 0;
    if (b1 && kb > b1_pass_bytes(kind)) {
        // Long 1-bit K: bands are required for exactness (see b1_pass_bytes).
        p.band = b1_band_bytes(kind, kb);
        if (variant == LB_AUTO) {
            // An automatic choice may cut K finer still (few tiles, see below).
            variant = resolve(dtype, LB_AUTO, M, N, K, cu);
            int64_t finer = kb;
            if (plan_ksplit(kind, variant, M, N, kb, cu, &finer) > 1 && finer < p.band) p.band = finer;
        }
        p.zero = true;
        p.parts[0].variant = variant;
    } else if (variant == LB_AUTO) {
        const int v = prefer_full_narrow_round(kind, resolve(dtype, LB_AUTO, M, N, K, cu), M, N, cu);
        p.np = plan_parts(dtype, v, M, N, K, cu, p.parts);
        if (p.np == 1 && plan_ksplit(kind, v, M, N, kb, cu, &p.band) > 1)
            p.zero = true;
        else if (p.np == 1)
            p.parts[0].variant = narrow_w4_tile(kind, v, M, N, cu);
    }
    return p;
}

int run_gemm(int kind, int dtype, int variant, const void *A, const void *B, void *out,
             size_t out_elem, const float *sx, const float *sw, int64_t M, int64_t N, int64_t K,
             int64_t kb, void *stream)
{
    const Plan p = make_plan(kind, dtype, variant, M, N, K, kb, 0);
    if (p.zero) {
        const hipError_t z = lb::launch_zero_i32((int32_t *)out, M * N, (hipStream_t)stream);
        if (z != hipSuccess) return LB_ERR_HIP;
    }
    for (int i = 0; i < p.np; ++i) {
        const Part &q = p.parts[i];
        const hipError_t e = lb::launch_mfma(
            kind, q.variant, (const int8_t *)A + q.m0 * kb, (const int8_t *)B + q.n0 * kb,
            (char *)out + (q.m0 * N + q.n0) * (int64_t)out_elem, sx ? sx + q.m0 : nullptr,
            sw ? sw + q.n0 : nullptr, q.m, q.n, kb, N, p.np == 1 ? p.band : kb, (hipStream_t)stream);
        if (e != hipSuccess) return LB_ERR_HIP;
    }
    return LB_OK;
}

}  // namespace

extern "C" {

int lb_gemm_s8(const int8_t *A, const int8_t *B, int32_t *C, int64_t M, int64_t N, int64_t K,
               int variant, void *stream)
{
    int st = check_common(A, B, C, M, N, K, LB_S8_K_ALIGN, LB_S8_K_MAX, variant);
    if (st != LB_OK) return st;
    return run_gemm(lb::KIND_S8, LB_S8, variant, A, B, C, 4, nullptr, nullptr, M, N, K, K, stream);
}

int lb_gemm_s4(const uint8_t *A, const uint8_t *B, int32_t *C, int64_t M, int64_t N, int64_t K,
               int variant, void *stream)
{
    int st = check_common(A, B, C, M, N, K, LB_S4_K_ALIGN, LB_S4_K_MAX, variant);
    if (st != LB_OK) return st;
    return run_gemm(lb::KIND_S4, LB_S4, variant, A, B, C, 4, nullptr, nullptr, M, N, K, K / 2, stream);
}

int lb_gemm_b1(const uint32_t *A, const uint32_t *B, int32_t *C, int64_t M, int64_t N, int64_t K,
               int variant, void *stream)
{
    int st = check_common(A, B, C, M, N, K, LB_B1_K_ALIGN, LB_B1_K_MAX, variant);
    if (st != LB_OK) return st;
    return run_gemm(b1_kind(), LB_B1, variant, A, B, C, 4, nullptr, nullptr, M, N, K, K / 8, stream);
}

int lb_auto_plan(int op, int64_t M, int64_t N, int64_t K, int cu_count, int *launches, int *tile_m,
                 int *tile_n, int *k_bands)
{
    if (M <= 0 || N <= 0 || K <= 0) return LB_ERR_SHAPE;
    int kind, dtype = op;
    int64_t kb;
    switch (op) {
    case LB_S8: kind = lb::KIND_S8; kb = K; break;
    case LB_S4: kind = lb::KIND_S4; kb = K / 2; break;
    case LB_B1: kind = b1_kind(); kb = K / 8; break;
    case LB_PLAN_LINEAR: kind = lb::KIND_LINEAR; dtype = LB_S8; kb = K; break;
    default: return LB_ERR_VARIANT;
    }
    if (kb <= 0) return LB_ERR_SHAPE;
    const Plan p = make_plan(kind, dtype, LB_AUTO, M, N, K, kb, cu_count);
    int bm = 0, bn = 0, bk = 0, st = 0;
    if (lb::mfma_variant_info(kind, p.parts[0].variant, &bm, &bn, &bk, &st) != 0) return LB_ERR_VARIANT;
    if (launches) *launches = p.np;
    if (tile_m) *tile_m = bm;
    if (tile_n) *tile_n = bn;
    if (k_bands) *k_bands = p.np == 1 ? (int)((kb + p.band - 1) / p.band) : 1;
    return LB_OK;
}

int lb_gemm_s8_linear(const int8_t *X, const int8_t *W, const float *sx, const float *sw,
                      float *out, int64_t M, int64_t N, int64_t K, int variant, void *stream)
{
    if (!sx || !sw) return LB_ERR_NULL;
    int st = check_common(X, W, out, M, N, K, LB_S8_K_ALIGN, LB_S8_K_MAX, variant);
    if (st != LB_OK) return st;
    return run_gemm(lb::KIND_LINEAR, LB_S8, variant, X, W, out, 4, sx, sw, M, N, K, K, stream);
}

}  // extern "C"

namespace {

// Shared checks and launch of the two convolutions.  kind selects int8 (C bytes
// per pixel) or int4 (C/2 bytes); calign is the channel rule, kmax the K limit.
int conv_entry(int kind, int dtype, const void *X, const void *F, int32_t *Y, int64_t N, int64_t H,
               int64_t W, int64_t C, int64_t Co, int64_t Kh, int64_t Kw, int64_t sh, int64_t sw,
               int64_t ph, int64_t pw, int variant, void *stream, int64_t calign, int64_t kmax)
{
    if (!X || !F || !Y) return LB_ERR_NULL;
    if (N <= 0 || H <= 0 || W <= 0 || C <= 0 || Co <= 0 || Kh <= 0 || Kw <= 0 || sh <= 0 ||
        sw <= 0 || ph < 0 || pw < 0)
        return LB_ERR_SHAPE;
    const int64_t lim = 0x7FFFFFFF;
    if (H > lim || W > lim || C > lim || Co > lim || Kh > lim || Kw > lim || sh > lim ||
        sw > lim || ph > lim || pw > lim)
        return LB_ERR_SHAPE;
    if (H + 2 * ph < Kh || W + 2 * pw < Kw) return LB_ERR_SHAPE;
    if (C % calign != 0) return LB_ERR_ALIGN;
    if (variant < LB_AUTO || variant >= LB_NUM_VARIANTS) return LB_ERR_VARIANT;
    const int64_t Ho = (H + 2 * ph - Kh) / sh + 1, Wo = (W + 2 * pw - Kw) / sw + 1;
    const int64_t cb = kind == lb::KIND_S8 ? C : C / 2;
    const int64_t K = Kh * Kw * C;  // elements per window
    if (K > kmax) return LB_ERR_OVERFLOW;
    // 32-bit byte offsets reach every pixel of the padded image and every output row.
    const double padded = (double)N * (double)(H + 2 * ph) * (double)(W + 2 * pw) * (double)cb;
    if (padded >= 2147483648.0 || (double)N * (double)Ho * (double)Wo >= 2147483648.0)
        return LB_ERR_OVERFLOW;
    const int64_t M = N * Ho * Wo, Kb = Kh * Kw * cb;
    // LB_AUTO: the variant the GEMM of the same M, N, K gets, except that a
    // layer with at most 64 output channels (N fits one small tile) takes the
    // small 2-stage tile.  Measured on MI355X over 12 layers with 32-128 output
    // channels: the small tile was the fastest in all 10 with Co <= 64, by
    // 0-29% over the GEMM's choice (int8 3x3 over 32 x 56x56x64 -> 64: 16.2
    // against 19.6 us; a 7x7 stride-2 stem: 72.9 against 89.1 us), the window
    // gather of a wider tile costing more than its column reuse saves; with 96
    // or 128 the GEMM's choice was within 3.4% of the best.  With windows of
    // several taps and at most 1024 bytes the same 64x64 tile runs with two
    // 64-byte stages instead (16 KiB of LDS: eight workgroups per CU against
    // five), since such layers are many short workgroups and what pays is how
    // many a CU holds.  Measured in one process against variant 0 (identical
    // results): int4 1.12-1.18x (7x7 stride-2 stem over 32 x 224x224x32 79.8
    // against 89.4 us, 3x3 over 8 x 112x112x32 12.1 against 14.3 us); int8
    // 0.99-1.12x (3x3 over 8 x 112x112x32 12.7 against 14.2 us, the stem
    // 73.4 against 72.9 us); a 1x1 layer lost 4% and windows of 1152 bytes
    // (3x3 over 28x28x128) 18% in an earlier build, so those keep variant 0.
    int v = variant;
    if (v == LB_AUTO && (v = auto_override()) < 0) {
        if (Co <= 64) v = (Kb <= 1024 && Kh * Kw > 1) ? lb::CONV_64x64_K64 : 0;
        else if (lb::select_from_table(dtype, M, Co, K, 0, &v, nullptr) != LB_OK) v = LB_DEFAULT_VARIANT;
    }
    lb::ConvGeom g;
    g.H = (int32_t)H; g.W = (int32_t)W; g.Cb = (int32_t)cb; g.Kh = (int32_t)Kh; g.Kw = (int32_t)Kw;
    g.sh = (int32_t)sh; g.sw = (int32_t)sw; g.ph = (int32_t)ph; g.pw = (int32_t)pw;
    g.Ho = (int32_t)Ho; g.Wo = (int32_t)Wo;
    g.x_bytes = (uint32_t)(N * H * W * cb);
    return finish(lb::launch_conv(kind, v, X, F, Y, M, Co, Kb, g, (hipStream_t)stream));
}

}  // namespace

extern "C" {

int lb_conv2d_s8(const int8_t *X, const int8_t *F, int32_t *Y, int64_t N, int64_t H, int64_t W,
                 int64_t C, int64_t Co, int64_t Kh, int64_t Kw, int64_t sh, int64_t sw, int64_t ph,
                 int64_t pw, int variant, void *stream)
{
    return conv_entry(lb::KIND_S8, LB_S8, X, F, Y, N, H, W, C, Co, Kh, Kw, sh, sw, ph, pw, variant,
                      stream, LB_CONV_S8_C_ALIGN, LB_S8_K_MAX);
}

int lb_conv2d_s4(const uint8_t *X, const uint8_t *F, int32_t *Y, int64_t N, int64_t H, int64_t W,
                 int64_t C, int64_t Co, int64_t Kh, int64_t Kw, int64_t sh, int64_t sw, int64_t ph,
                 int64_t pw, int variant, void *stream)
{
    return conv_entry(lb::KIND_S4, LB_S4, X, F, Y, N, H, W, C, Co, Kh, Kw, sh, sw, ph, pw, variant,
                      stream, LB_CONV_S4_C_ALIGN, LB_S4_K_MAX);
}

int lb_select_variant(int dtype, int64_t M, int64_t N, int64_t K, int cu_count, int *best,
                      int *second)
{
    if (!best) return LB_ERR_NULL;
    if (M <= 0 || N <= 0 || K <= 0) return LB_ERR_SHAPE;
    if (dtype != LB_S8 && dtype != LB_S4 && dtype != LB_B1) return LB_ERR_VARIANT;
    return lb::select_from_table(dtype, M, N, K, cu_count, best, second);
}

const char *lb_build_id(void) { return kBuildMark + 14; }

const char *lb_status_string(int status)
{
    switch (status) {
    case LB_OK: return "ok";
    case LB_ERR_NULL: return "null pointer";
    case LB_ERR_SHAPE: return "non-positive or too large M, N or K";
    case LB_ERR_ALIGN: return "K violates the alignment rule for this type";
    case LB_ERR_VARIANT: return "variant or dtype out of range";
    case LB_ERR_OVERFLOW: return "K above the limit for this type (the exact int32 sum must fit), "
                                 "or a convolution beyond 32-bit byte offsets";
    case LB_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

int lb_variant_info(int dtype, int variant, int *tile_m, int *tile_n, int *tile_k, int *stages)
{
    if (!tile_m || !tile_n || !tile_k || !stages) return LB_ERR_NULL;
    if (variant < 0 || variant >= LB_NUM_VARIANTS) return LB_ERR_VARIANT;
    int bk = 0;
    switch (dtype) {
    case LB_S8:
        if (lb::mfma_variant_info(lb::KIND_S8, variant, tile_m, tile_n, &bk, stages)) return LB_ERR_VARIANT;
        *tile_k = bk;
        return LB_OK;
    case LB_S4:
        if (lb::mfma_variant_info(lb::KIND_S4, variant, tile_m, tile_n, &bk, stages)) return LB_ERR_VARIANT;
        *tile_k = 2 * bk;
        return LB_OK;
    case LB_B1:
        if (lb::mfma_variant_info(lb::KIND_B1, variant, tile_m, tile_n, &bk, stages)) return LB_ERR_VARIANT;
        *tile_k = 8 * bk;
        return LB_OK;
    default: return LB_ERR_VARIANT;
    }
}

}  // extern "C"
