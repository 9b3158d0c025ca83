// lb_abi.cpp -- the extern "C" boundary declared in include/lb_gemm.h:
// argument checks, variant selection and launch on the caller's stream.
#include "lb_gemm.h"

#include <hip/hip_runtime.h>

#include "lb_internal.hpp"

namespace {

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

int resolve(int dtype, int variant, int64_t M, int64_t N, int64_t K)
{
    if (variant != LB_AUTO) return variant;
    int best = LB_DEFAULT_VARIANT;
    // cu_count 0: ask the current device; any failure keeps the default.
    if (lb::select_from_table(dtype, M, N, K, 0, &best, nullptr) != LB_OK) return LB_DEFAULT_VARIANT;
    return best;
}

int finish(hipError_t e) { return e == hipSuccess ? LB_OK : LB_ERR_HIP; }

}  // namespace

extern "C" {

int lb_gemm_s8(const int8_t *A, const int8_t *B, int32_t *C, int64_t M, int64_t N, int64_t K,
               int variant, void *stream)
{
    int st = check_common(A, B, C, M, N, K, LB_S8_K_ALIGN, LB_S8_K_MAX, variant);
    if (st != LB_OK) return st;
    const int v = resolve(LB_S8, variant, M, N, K);
    return finish(lb::launch_mfma(lb::KIND_S8, v, A, B, C, nullptr, nullptr, M, N, K,
                                  (hipStream_t)stream));
}

int lb_gemm_s4(const uint8_t *A, const uint8_t *B, int32_t *C, int64_t M, int64_t N, int64_t K,
               int variant, void *stream)
{
    int st = check_common(A, B, C, M, N, K, LB_S4_K_ALIGN, LB_S4_K_MAX, variant);
    if (st != LB_OK) return st;
    const int v = resolve(LB_S4, variant, M, N, K);
    return finish(lb::launch_mfma(lb::KIND_S4, v, A, B, C, nullptr, nullptr, M, N, K / 2,
                                  (hipStream_t)stream));
}

int lb_gemm_b1(const uint32_t *A, const uint32_t *B, int32_t *C, int64_t M, int64_t N, int64_t K,
               int variant, void *stream)
{
    int st = check_common(A, B, C, M, N, K, LB_B1_K_ALIGN, LB_B1_K_MAX, variant);
    if (st != LB_OK) return st;
    const int v = resolve(LB_B1, variant, M, N, K);
    return finish(lb::launch_b1(v, A, B, C, M, N, K / 32, (hipStream_t)stream));
}

int lb_gemm_s8_linear(const int8_t *X, const int8_t *W, const float *sx, const float *sw,
                      float *out, int64_t M, int64_t N, int64_t K, int variant, void *stream)
{
    if (!sx || !sw) return LB_ERR_NULL;
    int st = check_common(X, W, out, M, N, K, LB_S8_K_ALIGN, LB_S8_K_MAX, variant);
    if (st != LB_OK) return st;
    const int v = resolve(LB_S8, variant, M, N, K);
    return finish(lb::launch_mfma(lb::KIND_LINEAR, v, X, W, out, sx, sw, M, N, K,
                                  (hipStream_t)stream));
}

int lb_select_variant(int dtype, int64_t M, int64_t N, int64_t K, int cu_count, int *best,
                      int *second)
{
    if (!best) return LB_ERR_NULL;
    if (M <= 0 || N <= 0 || K <= 0) return LB_ERR_SHAPE;
    if (dtype != LB_S8 && dtype != LB_S4 && dtype != LB_B1) return LB_ERR_VARIANT;
    return lb::select_from_table(dtype, M, N, K, cu_count, best, second);
}

const char *lb_status_string(int status)
{
    switch (status) {
    case LB_OK: return "ok";
    case LB_ERR_NULL: return "null pointer";
    case LB_ERR_SHAPE: return "non-positive or too large M, N or K";
    case LB_ERR_ALIGN: return "K violates the alignment rule for this type";
    case LB_ERR_VARIANT: return "variant or dtype out of range";
    case LB_ERR_OVERFLOW: return "K above the limit for this type (exact int32 sum, or 1-bit addressing)";
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
        if (lb::mfma_variant_info(variant, tile_m, tile_n, &bk, stages)) return LB_ERR_VARIANT;
        *tile_k = bk;
        return LB_OK;
    case LB_S4:
        if (lb::mfma_variant_info(variant, tile_m, tile_n, &bk, stages)) return LB_ERR_VARIANT;
        *tile_k = 2 * bk;
        return LB_OK;
    case LB_B1:
        if (lb::b1_variant_info(variant, tile_m, tile_n, &bk, stages)) return LB_ERR_VARIANT;
        *tile_k = 32 * bk;
        return LB_OK;
    default: return LB_ERR_VARIANT;
    }
}

}  // extern "C"
