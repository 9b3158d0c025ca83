/*
 * lb_gemm.h -- exact low-bit integer GEMM for AMD MI355X (gfx950).
 *
 * The operation is the one stated in the digest of "Leveraging Large-Scale Data
 * for Efficient Low-Bit CUTLASS GEMM Optimization via Neural Networks" (IEEE
 * Transactions on Big Data): the matrix product A x B = C for 1-, 4- and 8-bit
 * operands, computed by a thread-block-tiled kernel whose tile shape and
 * pipeline depth are chosen per problem (Research results, items 1 and 2), and
 * used inside a low-bit linear layer (Research results, item 4).  Here every
 * product is accumulated exactly in int32.
 *
 * Plain C: loadable with dlopen/ctypes without HIP headers.
 *
 * Conventions shared by every call
 * --------------------------------
 * Layout (a reading; the pages fix only A x B = C):
 *   A    M x K, row-major: row m holds a(m, 0..K-1) contiguously.
 *   B    K x N, column-major: column n holds b(0..K-1, n) contiguously; these
 *        are the same bytes as an N x K row-major matrix (an nn.Linear weight).
 *   C    M x N, row-major, int32.  No leading-dimension arguments: every
 *        operand is dense.
 * Packing along K:
 *   int8  one signed byte per element, values -128..127.
 *   int4  two signed nibbles per byte (-8..7), even k in the low nibble.
 *   1-bit 32 elements per uint32, element k in bit (k % 32) of word k / 32;
 *         the product of two bits is their AND.
 * Pointers: device pointers (HBM) owned by the caller, readable/writable by the
 *   current HIP device.  Rows of A and B must start 16-byte aligned, which the
 *   alignment rule on K below guarantees for a 16-byte-aligned base (hipMalloc
 *   and torch give 256-byte-aligned bases).  The library does not allocate,
 *   free, copy or synchronise.
 * stream: a hipStream_t passed as void*; NULL is the null stream.  Calls are
 *   asynchronous: a status of LB_OK means the kernel was launched; a fault in
 *   the kernel surfaces at the caller's next synchronisation.
 * variant: 0..8 picks a kernel variant, index = 3*tile + (stages - 2) with tile
 *   0 = small, 1 = medium, 2 = large and stages 2, 3 or 4 (the nine templates:
 *   three tile sizes times three pipeline depths, Research results, item 2);
 *   LB_AUTO lets lb_select_variant choose for (dtype, M, N, K).  For the GEMMs
 *   and the linear layer, when that choice is a large-tile variant (one
 *   workgroup per CU) whose last round of tiles would fill at most half the
 *   CUs, LB_AUTO runs the product as two launches on the stream: the widest
 *   band of leading columns (else rows) of C that fills whole rounds, then the
 *   rest with the variant chosen for its own shape.  For the integer GEMMs,
 *   when the chosen variant's tiles fill at most a quarter of the CUs and K is
 *   long, LB_AUTO zeroes C with a kernel and cuts K into bands that add their
 *   exact partial sums into C.  For the int8 and int4 GEMMs and the linear
 *   layer, when the choice is variant 6 and neither applies but its 256x256
 *   tiles would fill less than one round of the CUs, LB_AUTO runs the same
 *   four-wave kernel on 256x192 tiles (int8 and linear: or 192x256) if those
 *   still fit in one round; and where such a round of narrower tiles would
 *   fill at least 7/8 of the CUs, LB_AUTO takes variant 6 for it whatever the
 *   selector chose (not when LB_AUTO_VARIANT fixes the variant).
 *   Either way the result is the same (integer sums do not depend on their
 *   order; the linear layer's dequantisation is per element); only the
 *   launches differ (lb_auto_plan reports them).  The
 *   environment variable LB_AUTO_VARIANT, set to one digit 0..8, replaces the
 *   selector's choice for every LB_AUTO call (GEMMs, linear layer and
 *   convolutions) and keeps the splits above: for tuning and tests.  Any other
 *   value is ignored.
 * Errors: every call returns an lb_status and never aborts.  Checks run in this
 *   order, before any HIP call: null pointer, non-positive size, K alignment,
 *   variant range, K limit; then the launch itself (LB_ERR_HIP).
 * Thread safety: calls may come from any thread; the shared state is the
 *   read-only selection table and a per-device cache of the CU count; each
 *   thread keeps its own memory of recent selections.
 */
#ifndef LB_GEMM_H
#define LB_GEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LB_OK = 0,
    LB_ERR_NULL = 1,     /* a required pointer is NULL */
    LB_ERR_SHAPE = 2,    /* M, N or K is not positive */
    LB_ERR_ALIGN = 3,    /* K violates the per-type alignment rule */
    LB_ERR_VARIANT = 4,  /* variant outside LB_AUTO..8, or dtype unknown */
    LB_ERR_OVERFLOW = 5, /* K above the type's limit (the exact int32 sum must fit);
                            convolutions: also 32-bit offset range */
    LB_ERR_HIP = 6       /* the HIP runtime reported an error */
} lb_status;

typedef enum { LB_S8 = 0, LB_S4 = 1, LB_B1 = 2 } lb_dtype;

#define LB_AUTO (-1)
#define LB_NUM_VARIANTS 9
#define LB_DEFAULT_VARIANT 7 /* large tile, 3 stages */

/* K limits: rows must be whole 16-byte chunks, and the worst-case |sum| must
 * fit int32 (16384 * K for int8; the int4 path accumulates 256 * a * b, the
 * same bound).  A 1-bit count never exceeds K, but one pass of the 1-bit
 * kernels accumulates 64 per matching bit pair (each bit position is weighted
 * so that a pair contributes 64 whatever its place in the byte), so a pass
 * covers at most 33,554,304 bits.  A longer 1-bit K (any variant) runs as K
 * bands of at most that many bits: C is zeroed by a fill kernel on the stream
 * and every band adds its exact counts into C with atomic adds.  The 1-bit
 * limit itself comes from 32-bit byte offsets inside a 256-row tile of A or
 * B: 255 rows of K/8 bytes must stay below 2^32, i.e. K < 2^27. */
#define LB_S8_K_ALIGN 16
#define LB_S4_K_ALIGN 32
#define LB_B1_K_ALIGN 128
#define LB_S8_K_MAX 131071
#define LB_S4_K_MAX 131071
#define LB_B1_K_MAX 134217600 /* largest multiple of 128 below 2^27 */

/*
 * C = A x B, int8 operands, int32 result.
 *   A: M*K int8 (row-major), B: N*K int8 (column-major K x N), C: M*N int32.
 *   K: elements (= bytes) per row; K % 16 == 0 and K <= LB_S8_K_MAX.
 */
int lb_gemm_s8(const int8_t *A, const int8_t *B, int32_t *C,
               int64_t M, int64_t N, int64_t K, int variant, void *stream);

/*
 * C = A x B, signed int4 operands packed two per byte, int32 result.
 *   A: M*K/2 bytes, B: N*K/2 bytes, C: M*N int32.
 *   K: int4 elements per row; K % 32 == 0 and K <= LB_S4_K_MAX.
 */
int lb_gemm_s4(const uint8_t *A, const uint8_t *B, int32_t *C,
               int64_t M, int64_t N, int64_t K, int variant, void *stream);

/*
 * C[m,n] = number of k with bit k set in both row m of A and column n of B.
 *   A: M*K/32 uint32, B: N*K/32 uint32, C: M*N int32.
 *   K: bits per row; K % 128 == 0 and K <= LB_B1_K_MAX.
 */
int lb_gemm_b1(const uint32_t *A, const uint32_t *B, int32_t *C,
               int64_t M, int64_t N, int64_t K, int variant, void *stream);

/*
 * Low-bit linear layer (Research results, item 4): int8 GEMM with the int32
 * accumulator dequantised in the epilogue, never written to memory:
 *   out[m*N+n] = ((float)acc[m,n] * sx[m]) * sw[n], fp32, round-to-nearest.
 *   X: M*K int8 activations (row-major), W: N*K int8 weights (column-major
 *   K x N, i.e. nn.Linear's [N, K]), sx: M fp32 per-row scales, sw: N fp32
 *   per-column scales, out: M*N fp32 (row-major).  K as for lb_gemm_s8.
 */
int lb_gemm_s8_linear(const int8_t *X, const int8_t *W, const float *sx,
                      const float *sw, float *out, int64_t M, int64_t N,
                      int64_t K, int variant, void *stream);

/*
 * Low-bit 2-D convolution over a batch of NHWC images (the im2win convolution
 * summary, gist.science paper 2608.20725: problem statement and method, which
 * treat the convolution layer over NHWC data for the whole batch at once).
 * The page gives no formula; this is the plain deep-learning convolution
 * (cross-correlation, zero padding, no dilation, groups or bias):
 *   Ho = (H + 2*ph - Kh)/sh + 1,  Wo = (W + 2*pw - Kw)/sw + 1,
 *   Y[((n*Ho + ho)*Wo + wo)*Co + co] = sum over kh < Kh, kw < Kw, c < C of
 *       X[n, ho*sh + kh - ph, wo*sw + kw - pw, c] * F[co, kh, kw, c]
 *   with X read as 0 outside the H x W image.
 *   X: N x H x W x C (NHWC), F: Co x Kh x Kw x C (channels innermost, i.e. Co
 *   rows of one window each), Y: N x Ho x Wo x Co int32 (NHWC).
 * It runs as a GEMM with M = N*Ho*Wo, N = Co, K = Kh*Kw*C whose A rows (the
 * page's windows) are read straight from X: no window or column buffer is
 * allocated.  LB_AUTO picks the variant the GEMM of that shape would get, or
 * when Co <= 64 the small 64x64 tile: with two 64-byte stages (an internal
 * tile, up to eight workgroups per CU) when the filter has more than one tap
 * and a window holds at most 1024 bytes, else the 2-stage tile of variant 0.
 * C must be a multiple of LB_CONV_S8_C_ALIGN (int8) or LB_CONV_S4_C_ALIGN
 * (int4, packed two per byte along C, even c in the low nibble, for X and F
 * alike): 16 bytes per pixel or a multiple, else LB_ERR_ALIGN.  (A layer with
 * fewer channels, e.g. an RGB input, runs with its channels zero-padded to 16
 * in X and F; the result is the same.)  LB_ERR_SHAPE for a non-positive size or stride,
 * negative padding or a filter wider than the padded image; LB_ERR_OVERFLOW if
 * Kh*Kw*C exceeds the type's K limit or the padded image or N*Ho*Wo reaches
 * 2^31 (byte offsets are 32-bit).  Pointers, stream and errors otherwise as for
 * the GEMMs.
 */
#define LB_CONV_S8_C_ALIGN 16
#define LB_CONV_S4_C_ALIGN 32
int lb_conv2d_s8(const int8_t *X, const int8_t *F, int32_t *Y, int64_t N,
                 int64_t H, int64_t W, int64_t C, int64_t Co, int64_t Kh,
                 int64_t Kw, int64_t sh, int64_t sw, int64_t ph, int64_t pw,
                 int variant, void *stream);
int lb_conv2d_s4(const uint8_t *X, const uint8_t *F, int32_t *Y, int64_t N,
                 int64_t H, int64_t W, int64_t C, int64_t Co, int64_t Kh,
                 int64_t Kw, int64_t sh, int64_t sw, int64_t ph, int64_t pw,
                 int variant, void *stream);

/*
 * Per-shape variant choice (Research results, items 2-3: the template index is
 * predicted from M, N, K and the GPU's multiprocessor count, and judged by
 * whether the true best template is among the top two).
 *   dtype: an lb_dtype.  M, N, K as for the GEMM of that dtype (K in elements
 *   or bits).  cu_count: compute units of the target GPU; <= 0 queries the
 *   current HIP device.  best: receives the chosen variant (0..8).  second:
 *   receives the runner-up, or may be NULL.
 * By default the choice is the label of the nearest shape in a table of
 * timings measured on MI355X; with the environment variable LB_SELECTOR=mlp
 * the pages' feed-forward classifier (three hidden layers of 128) decides.
 * Host-only, microseconds, no GPU work.  Returns LB_ERR_NULL if best is NULL,
 * LB_ERR_SHAPE for non-positive sizes, LB_ERR_VARIANT for an unknown dtype and
 * LB_ERR_HIP if cu_count <= 0 and no device can be queried.
 */
int lb_select_variant(int dtype, int64_t M, int64_t N, int64_t K, int cu_count,
                      int *best, int *second);

/* The launches an LB_AUTO call makes for a shape, without launching anything
 * (host-only; for tests and tuning).  op: LB_S8, LB_S4 or LB_B1 for the GEMMs,
 * LB_PLAN_LINEAR for the int8 linear layer; M, N, K as for that call.
 * cu_count: compute units to plan for; <= 0 asks the current HIP device (if
 * none answers, the plan is the one a call would make without that
 * information: the default variant, no splits, bands or narrow tiles).
 * Writes, through any non-NULL pointer: launches (1, or 2 for the two-launch
 * split), tile_m x tile_n (the workgroup tile of the first launch: a
 * variant's tile, or 256 x 192 / 192 x 256, the four-wave kernel's narrower
 * tiles that an automatic choice of variant 6 takes when its 256x256 grid
 * would fill less than one round of the CUs and the narrower grid still fits
 * in one), and k_bands (K bands of a single launch; 1: none).  Returns
 * LB_ERR_SHAPE for a non-positive size (or K below one byte of the type),
 * LB_ERR_VARIANT for an unknown op. */
#define LB_PLAN_LINEAR 3
int lb_auto_plan(int op, int64_t M, int64_t N, int64_t K, int cu_count, int *launches,
                 int *tile_m, int *tile_n, int *k_bands);

/* Hash of the source files this library was built from (16 hex digits, static
 * storage; never NULL).  The build stamps it in, so that a caller can check a
 * loaded library against the sources it expects. */
const char *lb_build_id(void);

/* Human-readable name of a status code (static storage; never NULL). */
const char *lb_status_string(int status);

/* Tile and stage description of a variant for a dtype: writes the workgroup
 * tile (rows of C, columns of C, K elements per pipeline stage) and the stage
 * count.  Returns LB_ERR_VARIANT for an index outside 0..8 or unknown dtype. */
int lb_variant_info(int dtype, int variant, int *tile_m, int *tile_n,
                    int *tile_k, int *stages);

#ifdef __cplusplus
}
#endif

#endif /* LB_GEMM_H */
