/*
 * oracle.c -- plain, slow, obviously correct CPU reference for the low-bit
 * integer GEMM.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the
 * CPU-baseline leg of the benchmark call it; the GPU library never does, and
 * this file shares no code, header, table or helper with it.
 *
 * What is computed.  The digest of "Leveraging Large-Scale Data for Efficient
 * Low-Bit CUTLASS GEMM Optimization via Neural Networks" (IEEE Transactions on
 * Big Data) states the problem as the matrix product A x B = C split into
 * thread-block tiles along M and N with a loop over K (Research results, item 1:
 * the customisable GEMM template and its optimisation space), for operands of
 * 1, 4 and 8 bits (editor's summary and the methods paragraph that lists the
 * three data types of the dataset).  The product is exact, so this oracle is
 * the definition written out: one multiply-add per (m, n, k), no blocking, no
 * reordering, accumulated in 64-bit integers and then checked to fit int32.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - 8-bit operands are signed int8 in [-128, 127].
 *   - 4-bit operands are signed two's-complement nibbles in [-8, 7], packed two
 *     per byte along K with the even k in the low nibble.
 *   - 1-bit operands are {0, 1} packed 32 per uint32 along K, bit (k mod 32) of
 *     word (k / 32) holding element k; the product of two bits is their AND.
 *   - A is M x K row-major; B is K x N column-major, i.e. N rows of K values;
 *     C is M x N row-major int32.
 *   - The linear layer (Research results, item 4, names a linear layer built on
 *     the selected GEMM) dequantises with one scale per row of X and one per
 *     output column: out = acc * sx[m] * sw[n].  The oracle evaluates it in
 *     fp64, which the GPU's fp32 result must match to 1e-6 relative.
 *
 * Every function returns 0 on success and 1 if some exact sum falls outside
 * int32 (the result buffer then holds the low 32 bits of those sums, and the
 * caller must treat it as invalid); the convolutions return 2 for impossible
 * geometry (non-positive stride, negative padding, window wider than the
 * padded image).  Shapes must be positive; K must be a
 * multiple of 2 (int4) or 32 (1-bit) so that rows hold whole bytes / words.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC (no intrinsics, no
 * BLAS).  OpenMP splits the outer loop over rows of C only.
 */
#include <stdint.h>

/* ---- element decoders: one value of row `row`, column k ------------------ */

static int s8_at(const int8_t *rowp, int64_t k) { return (int)rowp[k]; }

/* Signed nibble: even k in bits 0..3, odd k in bits 4..7 of byte k/2. */
static int s4_at(const uint8_t *rowp, int64_t k)
{
    unsigned byte = rowp[k / 2];
    unsigned nib = (k % 2 == 0) ? (byte & 0xFu) : ((byte >> 4) & 0xFu);
    return (nib >= 8u) ? (int)nib - 16 : (int)nib;
}

/* Bit k of the row: word k/32, bit position k%32 (least significant = lowest k). */
static int b1_at(const uint32_t *rowp, int64_t k)
{
    return (int)((rowp[k / 32] >> (k % 32)) & 1u);
}

static int fits_i32(int64_t v) { return v >= INT32_MIN && v <= INT32_MAX; }

/* ---- GEMMs: C[m*N+n] = sum_k a(m,k) * b(n,k) ------------------------------ */

int orc_gemm_s8(const int8_t *A, const int8_t *B, int32_t *C,
                int64_t M, int64_t N, int64_t K)
{
    int bad = 0;
    int64_t m;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (m = 0; m < M; ++m) {
        const int8_t *arow = A + m * K;
        for (int64_t n = 0; n < N; ++n) {
            const int8_t *brow = B + n * K;
            int64_t acc = 0;
            for (int64_t k = 0; k < K; ++k)
                acc += (int64_t)s8_at(arow, k) * (int64_t)s8_at(brow, k);
            if (!fits_i32(acc)) bad = 1;
            C[m * N + n] = (int32_t)(uint32_t)(uint64_t)acc;
        }
    }
    return bad;
}

int orc_gemm_s4(const uint8_t *A, const uint8_t *B, int32_t *C,
                int64_t M, int64_t N, int64_t K)
{
    int bad = 0;
    const int64_t row_bytes = K / 2;
    int64_t m;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (m = 0; m < M; ++m) {
        const uint8_t *arow = A + m * row_bytes;
        for (int64_t n = 0; n < N; ++n) {
            const uint8_t *brow = B + n * row_bytes;
            int64_t acc = 0;
            for (int64_t k = 0; k < K; ++k)
                acc += (int64_t)s4_at(arow, k) * (int64_t)s4_at(brow, k);
            if (!fits_i32(acc)) bad = 1;
            C[m * N + n] = (int32_t)(uint32_t)(uint64_t)acc;
        }
    }
    return bad;
}

/* 1-bit: the product of two {0,1} elements, summed over every bit position. */
int orc_gemm_b1(const uint32_t *A, const uint32_t *B, int32_t *C,
                int64_t M, int64_t N, int64_t K)
{
    int bad = 0;
    const int64_t row_words = K / 32;
    int64_t m;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (m = 0; m < M; ++m) {
        const uint32_t *arow = A + m * row_words;
        for (int64_t n = 0; n < N; ++n) {
            const uint32_t *brow = B + n * row_words;
            int64_t acc = 0;
            for (int64_t k = 0; k < K; ++k)
                acc += (int64_t)(b1_at(arow, k) * b1_at(brow, k));
            if (!fits_i32(acc)) bad = 1;
            C[m * N + n] = (int32_t)(uint32_t)(uint64_t)acc;
        }
    }
    return bad;
}

/* ---- linear layer: int8 GEMM, then per-row x per-column dequantisation ---- */

int orc_linear_s8(const int8_t *X, const int8_t *W, const float *sx,
                  const float *sw, double *out, int64_t M, int64_t N, int64_t K)
{
    int bad = 0;
    int64_t m;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (m = 0; m < M; ++m) {
        const int8_t *xrow = X + m * K;
        for (int64_t n = 0; n < N; ++n) {
            const int8_t *wrow = W + n * K;
            int64_t acc = 0;
            for (int64_t k = 0; k < K; ++k)
                acc += (int64_t)s8_at(xrow, k) * (int64_t)s8_at(wrow, k);
            if (!fits_i32(acc)) bad = 1;
            out[m * N + n] = (double)acc * (double)sx[m] * (double)sw[n];
        }
    }
    return bad;
}

/* ---- 2-D convolution ------------------------------------------------------
 *
 * The im2win convolution summary (gist.science paper 2608.20725, "method":
 * data transformation, NHWC layout, whole-batch execution) treats the
 * convolution layer of a deep network: a window slides over each image and the
 * values under it are multiplied with a filter and summed.  The page fixes no
 * formula; the readings here (listed in the design notes) are the plain
 * deep-learning convolution, i.e. cross-correlation without flipping:
 *   x : N x H x W x C (NHWC)          f : Co x Kh x Kw x C (channels innermost)
 *   y : N x Ho x Wo x Co int32 (NHWC), Ho = (H + 2 ph - Kh) / sh + 1,
 *                                      Wo = (W + 2 pw - Kw) / sw + 1
 *   y[n,ho,wo,co] = sum over kh, kw, c of
 *                   x[n, ho*sh + kh - ph, wo*sw + kw - pw, c] * f[co, kh, kw, c]
 * with x taken as 0 outside the image (zero padding).  No dilation, groups or
 * bias.  The int4 variant packs two values per byte along C (even c in the low
 * nibble), for the image and the filter alike.
 *
 * orc_conv2d_* is that definition written out.  orc_im2win_s8 and
 * orc_conv2d_im2win_s8 follow the page's method instead: build the window
 * tensor, then take each output as one contiguous dot product.  The tests
 * require the two routes to agree. */

/* Element c of the pixel (n, h, w), or 0 outside the image. */
static int x8_at(const int8_t *X, int64_t H, int64_t W, int64_t C,
                 int64_t n, int64_t h, int64_t w, int64_t c)
{
    if (h < 0 || h >= H || w < 0 || w >= W) return 0;
    return s8_at(X + ((n * H + h) * W + w) * C, c);
}

static int x4_at(const uint8_t *X, int64_t H, int64_t W, int64_t C,
                 int64_t n, int64_t h, int64_t w, int64_t c)
{
    if (h < 0 || h >= H || w < 0 || w >= W) return 0;
    return s4_at(X + ((n * H + h) * W + w) * (C / 2), c);
}

static int conv_dims(int64_t H, int64_t W, int64_t Kh, int64_t Kw, int64_t sh,
                     int64_t sw, int64_t ph, int64_t pw, int64_t *Ho, int64_t *Wo)
{
    if (sh <= 0 || sw <= 0 || ph < 0 || pw < 0) return 1;
    if (H + 2 * ph < Kh || W + 2 * pw < Kw) return 1;
    *Ho = (H + 2 * ph - Kh) / sh + 1;
    *Wo = (W + 2 * pw - Kw) / sw + 1;
    return 0;
}

int orc_conv2d_s8(const int8_t *X, const int8_t *F, int32_t *Y, int64_t N, int64_t H,
                  int64_t W, int64_t C, int64_t Co, int64_t Kh, int64_t Kw, int64_t sh,
                  int64_t sw, int64_t ph, int64_t pw)
{
    int64_t Ho, Wo;
    if (conv_dims(H, W, Kh, Kw, sh, sw, ph, pw, &Ho, &Wo)) return 2;
    int bad = 0;
    int64_t q;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (q = 0; q < N * Ho; ++q) {
        const int64_t n = q / Ho, ho = q % Ho;
        for (int64_t wo = 0; wo < Wo; ++wo)
            for (int64_t co = 0; co < Co; ++co) {
                int64_t acc = 0;
                for (int64_t kh = 0; kh < Kh; ++kh)
                    for (int64_t kw = 0; kw < Kw; ++kw)
                        for (int64_t c = 0; c < C; ++c)
                            acc += (int64_t)x8_at(X, H, W, C, n, ho * sh + kh - ph, wo * sw + kw - pw, c) *
                                   (int64_t)s8_at(F + ((co * Kh + kh) * Kw + kw) * C, c);
                if (!fits_i32(acc)) bad = 1;
                Y[((n * Ho + ho) * Wo + wo) * Co + co] = (int32_t)(uint32_t)(uint64_t)acc;
            }
    }
    return bad;
}

int orc_conv2d_s4(const uint8_t *X, const uint8_t *F, int32_t *Y, int64_t N, int64_t H,
                  int64_t W, int64_t C, int64_t Co, int64_t Kh, int64_t Kw, int64_t sh,
                  int64_t sw, int64_t ph, int64_t pw)
{
    int64_t Ho, Wo;
    if (C % 2 || conv_dims(H, W, Kh, Kw, sh, sw, ph, pw, &Ho, &Wo)) return 2;
    int bad = 0;
    int64_t q;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (q = 0; q < N * Ho; ++q) {
        const int64_t n = q / Ho, ho = q % Ho;
        for (int64_t wo = 0; wo < Wo; ++wo)
            for (int64_t co = 0; co < Co; ++co) {
                int64_t acc = 0;
                for (int64_t kh = 0; kh < Kh; ++kh)
                    for (int64_t kw = 0; kw < Kw; ++kw)
                        for (int64_t c = 0; c < C; ++c)
                            acc += (int64_t)x4_at(X, H, W, C, n, ho * sh + kh - ph, wo * sw + kw - pw, c) *
                                   (int64_t)s4_at(F + ((co * Kh + kh) * Kw + kw) * (C / 2), c);
                if (!fits_i32(acc)) bad = 1;
                Y[((n * Ho + ho) * Wo + wo) * Co + co] = (int32_t)(uint32_t)(uint64_t)acc;
            }
    }
    return bad;
}

/* The window tensor of the page's data transformation.  For each image n and
 * output row ho, the Kh input rows that row ho reads are interleaved so that
 * every padded column w holds its Kh x C values next to each other:
 *   win[(((n*Ho + ho)*Wp + w)*Kh + kh)*C + c] = x[n, ho*sh + kh - ph, w - pw, c],
 * Wp = W + 2 pw.  Rows that windows of different outputs share are stored once
 * per output row, not once per output. */
int orc_im2win_s8(const int8_t *X, int8_t *Win, int64_t N, int64_t H, int64_t W, int64_t C,
                  int64_t Kh, int64_t Kw, int64_t sh, int64_t sw, int64_t ph, int64_t pw)
{
    int64_t Ho, Wo;
    if (conv_dims(H, W, Kh, Kw, sh, sw, ph, pw, &Ho, &Wo)) return 2;
    const int64_t Wp = W + 2 * pw;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t ho = 0; ho < Ho; ++ho)
            for (int64_t w = 0; w < Wp; ++w)
                for (int64_t kh = 0; kh < Kh; ++kh)
                    for (int64_t c = 0; c < C; ++c)
                        Win[(((n * Ho + ho) * Wp + w) * Kh + kh) * C + c] =
                            (int8_t)x8_at(X, H, W, C, n, ho * sh + kh - ph, w - pw, c);
    return 0;
}

/* Output (n, ho, wo) from the window tensor: its window is the contiguous run
 * of Kw*Kh*C values that starts at column w = wo*sw of row (n, ho), ordered
 * (kw, kh, c); the filter value for run position t is f[co, kh, kw, c]. */
int orc_conv2d_im2win_s8(const int8_t *Win, const int8_t *F, int32_t *Y, int64_t N, int64_t H,
                         int64_t W, int64_t C, int64_t Co, int64_t Kh, int64_t Kw, int64_t sh,
                         int64_t sw, int64_t ph, int64_t pw)
{
    int64_t Ho, Wo;
    if (conv_dims(H, W, Kh, Kw, sh, sw, ph, pw, &Ho, &Wo)) return 2;
    const int64_t Wp = W + 2 * pw, run = Kw * Kh * C;
    int bad = 0;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t ho = 0; ho < Ho; ++ho) {
            const int8_t *row = Win + (n * Ho + ho) * Wp * Kh * C;
            for (int64_t wo = 0; wo < Wo; ++wo) {
                const int8_t *window = row + wo * sw * Kh * C;
                for (int64_t co = 0; co < Co; ++co) {
                    int64_t acc = 0;
                    for (int64_t t = 0; t < run; ++t) {
                        const int64_t kw = t / (Kh * C), kh = (t / C) % Kh, c = t % C;
                        acc += (int64_t)window[t] * (int64_t)F[((co * Kh + kh) * Kw + kw) * C + c];
                    }
                    if (!fits_i32(acc)) bad = 1;
                    Y[((n * Ho + ho) * Wo + wo) * Co + co] = (int32_t)(uint32_t)(uint64_t)acc;
                }
            }
        }
    return bad;
}

/* Threads OpenMP will use for the loops above (reported with CPU timings). */
#ifdef _OPENMP
#include <omp.h>
int orc_num_threads(void) { return omp_get_max_threads(); }
#else
int orc_num_threads(void) { return 1; }
#endif
