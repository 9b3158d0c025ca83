// lb_internal.hpp -- host-side interface between the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lb {

// KIND_B1 runs the 1-bit GEMM on the int8 instruction (eight weighted bit
// planes per 64-byte block), KIND_B1F4 on the FP4 instruction (four bit planes
// per block, fp32 accumulation exact below 2^24).
enum { KIND_S8 = 0, KIND_S4 = 1, KIND_LINEAR = 2, KIND_B1 = 3, KIND_B1F4 = 4 };

// Internal tile codes beside the nine public variants (never accepted from a
// caller): the four-wave kernel on 256x192 tiles (int8, int4 and 1-bit FP4-
// route GEMMs, linear layer) and on 192x256 tiles (int8 GEMM, linear layer).
enum { W4_256x192 = 16, W4_192x256 = 17 };
// Internal tile code of the convolutions: a 64x64 tile with two 64-byte
// stages (16 KiB of LDS, up to eight workgroups per CU).
enum { CONV_64x64_K64 = 18 };

// int8 MFMA family (int8 GEMM, packed-int4 GEMM, int8 linear layer, and the
// 1-bit GEMM on weighted bit planes).  Kb is the row length of A and B in
// bytes (K for int8, K/2 for int4, K/8 for 1-bit); ldo is the distance in
// elements between rows of the output (N for a whole product, more when the
// launch covers a band of its columns).  ksplit < Kb (integer GEMMs only, a
// multiple of the variant's stage depth) runs ceil(Kb / ksplit) bands of K in
// one grid, each adding its partial sums into C, which must hold zeros.
hipError_t launch_mfma(int kind, int variant, const void *A, const void *B, void *out,
                       const float *sx, const float *sw, int64_t M, int64_t N, int64_t Kb,
                       int64_t ldo, int64_t ksplit, hipStream_t s);
// Zero n int32 values on the stream (a kernel, not a memset).
hipError_t launch_zero_i32(int32_t *p, int64_t n, hipStream_t s);
// Workgroup tile and stage of a variant; bk_bytes is the K depth of a stage in bytes.
int mfma_variant_info(int kind, int variant, int *bm, int *bn, int *bk_bytes, int *stages);

// Geometry of a convolution run as a GEMM whose A rows are gathered from an
// NHWC image: output pixel r = (n*Ho + ho)*Wo + wo is row r, the filter taps
// (kh, kw, channel byte) are the K axis.  Cb is bytes per pixel (C or C/2) and
// a multiple of 16; x_bytes = N*H*W*Cb < 2^31.
struct ConvGeom {
    int32_t H, W, Cb, Kh, Kw, sh, sw, ph, pw, Ho, Wo;
    uint32_t x_bytes;
};
// kind KIND_S8 or KIND_S4; M = N*Ho*Wo, N = Co, Kb = Kh*Kw*Cb.
hipError_t launch_conv(int kind, int variant, const void *X, const void *F, int32_t *Y,
                       int64_t M, int64_t N, int64_t Kb, const ConvGeom &g, hipStream_t s);

// Measured selection table lookup (host only).
int select_from_table(int dtype, int64_t M, int64_t N, int64_t K, int cu_count, int *best,
                      int *second);
// Compute units of the current device (cached per device).
int device_cu_count(int *cu);

}  // namespace lb
