// lb_internal.hpp -- host-side interface between the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lb {

enum { KIND_S8 = 0, KIND_S4 = 1, KIND_LINEAR = 2 };

// int8 MFMA family (int8 GEMM, packed-int4 GEMM, int8 linear layer).
// Kb is the row length of A and B in bytes (K for int8, K/2 for int4).
hipError_t launch_mfma(int kind, int variant, const void *A, const void *B, void *out,
                       const float *sx, const float *sw, int64_t M, int64_t N, int64_t Kb,
                       hipStream_t s);
int mfma_variant_info(int variant, int *bm, int *bn, int *bk_bytes, int *stages);

// 1-bit VALU family.  Kw is the row length in 32-bit words (K/32).
hipError_t launch_b1(int variant, const uint32_t *A, const uint32_t *B, int32_t *C, int64_t M,
                     int64_t N, int64_t Kw, hipStream_t s);
int b1_variant_info(int variant, int *bm, int *bn, int *bk_words, int *stages);

// Measured selection table lookup (host only).
int select_from_table(int dtype, int64_t M, int64_t N, int64_t K, int cu_count, int *best,
                      int *second);

}  // namespace lb
