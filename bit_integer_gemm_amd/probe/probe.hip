// probe.hip -- measurements behind design decisions of the low-bit GEMM (not
// part of the GEMM library).
//
// 1. Issue rate of the gfx950 matrix instructions a low-bit GEMM can run on, measured with realistic operand bits: int8 16x16x64 (uniform
// random bytes, the int8 GEMM), and the scaled 16x16x128 instruction with FP8
// e4m3, FP6 e3m2 (int4 values, which e3m2 holds exactly) and FP4 e2m1 (one
// bit per nibble, the 1-bit GEMM's bit planes) operands.  Each wave keeps 16
// independent accumulators, so the count is issue-bound, not latency-bound.
//
// 2. Write bandwidth of a GEMM-like output store when only some workgroups
// store at a time: every workgroup writes its own contiguous 256 KiB (a
// 256 x 256 int32 tile) with 16-byte stores, and a mask picks the ones that do
// (all of them; those of one XCD; or 1 in 8 of every XCD's).  Whether the
// store phase of a GEMM is bound per XCD or chip-wide decides whether
// staggering tiles in time can hide it.
//
// 3. (below) MFMA throughput with independent vector instructions between.
//
// 4. (below) Cycles per MFMA slot of one wave that issues V other instructions
// after each MFMA: the cost of a vector instruction placed between a wave's own
// MFMAs, which decides how the int4 and 1-bit plane unpack is spread.
//
// 5. (below) Cycles per MFMA of a wave that also issues direct global->LDS
// copies (16 bytes per lane) between its MFMAs, B copies after every CPM-th
// MFMA, in all four waves of a workgroup or in wave 0 only: the cost of a copy
// to its wave, and the CU's copy bandwidth once copies collide.
//
// 6. (below) The 1-bit GEMM on the vector ALUs, the form the scope of the
// 1-bit product starts from: each thread owns an 8 x 8 block of C and adds
// popcount(a AND b) of 32-bit words (one v_and_b32 and one v_bcnt_u32_b32 per
// word pair, 64 bit-MACs).  Its rate against the vector ALUs' peak, and
// against the library's matrix-core route, measured on the same shape.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x6 __attribute__((ext_vector_type(6)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

enum { R_I8 = 0, R_FP8 = 1, R_FP6 = 2, R_FP4 = 3 };

__device__ inline uint32_t mix(uint32_t x)
{
    x ^= x >> 16; x *= 0x7feb352dU; x ^= x >> 15; x *= 0x846ca68bU; x ^= x >> 16;
    return x;
}

// Operand bits for one lane: `words` 32-bit words in the instruction's format.
template <int KIND>
__device__ inline uint32_t operand_word(uint32_t s)
{
    const uint32_t r = mix(s);
    if constexpr (KIND == R_I8) return r;                          // any byte is an int8
    if constexpr (KIND == R_FP8) return r & 0x77777777u;           // e4m3 without NaN codes
    if constexpr (KIND == R_FP6) return r;                         // every e3m2 code is finite
    return r & 0x11111111u;                                        // e2m1 0.5 or 0: one bit plane
}

// The instructions are inline assembly with the accumulator tied to its
// AGPRs: with the builtins the compiler rotates accumulators between register
// files and pads the loop with moves and wait states, which it then measures.
template <int KIND>
__device__ inline void mma(f32x4 &acc, const i32x8 &a, const i32x8 &b, int one)
{
    if constexpr (KIND == R_FP8) {
        asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %3 op_sel_hi:[0,0,0]"
                     : "+a"(acc) : "v"(a), "v"(b), "v"(one));
    } else if constexpr (KIND == R_FP6) {
        const i32x6 a6 = {a[0], a[1], a[2], a[3], a[4], a[5]}, b6 = {b[0], b[1], b[2], b[3], b[4], b[5]};
        asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %3 op_sel_hi:[0,0,0] cbsz:3 blgp:3"
                     : "+a"(acc) : "v"(a6), "v"(b6), "v"(one));
    } else {
        const i32x4 a4 = {a[0], a[1], a[2], a[3]}, b4 = {b[0], b[1], b[2], b[3]};
        asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %3 op_sel_hi:[0,0,0] cbsz:4 blgp:4"
                     : "+a"(acc) : "v"(a4), "v"(b4), "v"(one));
    }
}

template <int KIND>
__global__ __launch_bounds__(256) void rate_kernel(uint32_t seed, int iters, float *out)
{
    const uint32_t gid = blockIdx.x * 256u + threadIdx.x;
    i32x8 a, b;
    for (int d = 0; d < 8; ++d) {
        a[d] = (int)operand_word<KIND>(seed ^ (gid * 16u + (uint32_t)d));
        b[d] = (int)operand_word<KIND>(seed ^ (gid * 16u + 8u + (uint32_t)d) ^ 0x5bd1e995u);
    }
    float total = 0.f;
    if constexpr (KIND == R_I8) {
        i32x4 acc[16];
        for (int q = 0; q < 16; ++q) acc[q] = i32x4{0, 0, 0, 0};
        const i32x4 a4 = {a[0], a[1], a[2], a[3]}, b4 = {b[0], b[1], b[2], b[3]};
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int q = 0; q < 16; ++q)
                asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+a"(acc[q]) : "v"(a4), "v"(b4));
        }
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
        for (int q = 0; q < 16; ++q) total += (float)(acc[q][0] + acc[q][1] + acc[q][2] + acc[q][3]);
    } else {
        f32x4 acc[16];
        for (int q = 0; q < 16; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int one = 127;  // E8M0 scale 2^0
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int q = 0; q < 16; ++q) mma<KIND>(acc[q], a, b, one);
        }
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
        for (int q = 0; q < 16; ++q) total += acc[q][0] + acc[q][1] + acc[q][2] + acc[q][3];
    }
    out[gid] = total;
}

// 3. Matrix core and vector ALU side by side: every int8 16x16x64 MFMA is
// followed by V independent vector instructions (v_xor_b32 on registers no
// MFMA reads).  If the two share one issue slot per SIMD, time per MFMA grows
// by the VALU issue time (4 cycles for a wave64 instruction on 16 lanes) as
// soon as V is large enough; if they run side by side, it stays flat while
// the vector work fits in the MFMA's own duration.
template <int V>
__global__ __launch_bounds__(256) void mix_kernel(uint32_t seed, int iters, float *out)
{
    const uint32_t gid = blockIdx.x * 256u + threadIdx.x;
    const i32x4 a = {(int)mix(seed ^ gid), (int)mix(seed + gid), (int)mix(seed * 3u + gid), (int)mix(gid)};
    const i32x4 b = {(int)mix(a[0]), (int)mix(a[1]), (int)mix(a[2]), (int)mix(a[3])};
    i32x4 acc[16];
    for (int q = 0; q < 16; ++q) acc[q] = i32x4{0, 0, 0, 0};
    uint32_t x0 = gid, x1 = gid * 7u, x2 = gid * 13u, x3 = gid * 29u;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+a"(acc[q]) : "v"(a), "v"(b));
            if constexpr (V >= 1) asm volatile("v_xor_b32 %0, 0x55, %0" : "+v"(x0));
            if constexpr (V >= 2) asm volatile("v_xor_b32 %0, 0x55, %0" : "+v"(x1));
            if constexpr (V >= 3) asm volatile("v_xor_b32 %0, 0x55, %0" : "+v"(x2));
            if constexpr (V >= 4) asm volatile("v_xor_b32 %0, 0x55, %0" : "+v"(x3));
        }
    }
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    float total = (float)(x0 ^ x1 ^ x2 ^ x3);
    for (int q = 0; q < 16; ++q) total += (float)(acc[q][0] + acc[q][1] + acc[q][2] + acc[q][3]);
    out[gid] = total;
}

// Workgroup b writes bytes [b * chunk, (b + 1) * chunk) of out when it is
// selected: mode 0 every workgroup, mode 1 those with b % 8 == 0 (consecutive
// workgroups go round robin over the 8 XCDs, so: the CUs of one XCD), mode 2
// those with (b / 8) % 8 == 0 (one in eight of every XCD's).
__global__ __launch_bounds__(256) void store_kernel(i32x4 *out, int chunk_vec, int mode)
{
    const uint32_t b = blockIdx.x;
    const bool on = mode == 0 || (mode == 1 && b % 8u == 0u) || (mode == 2 && (b / 8u) % 8u == 0u);
    if (!on) return;
    i32x4 *p = out + (size_t)b * (size_t)chunk_vec;
    const i32x4 v = {(int)b, (int)threadIdx.x, 1, 2};
    for (int i = threadIdx.x; i < chunk_vec; i += 256) p[i] = v;
}

// 4. OP 0: v_and_b32 with an SGPR mask (the unpack's masking), 1: 64-bit
// shift (v_lshlrev_b64), 2: s_nop 1; V instructions after each MFMA, on
// registers no MFMA reads.  Per-wave cycles (s_memtime) into cyc[wave].
template <int OP, int V>
__global__ __launch_bounds__(256) void slot_kernel(int iters, uint32_t msk, uint32_t *cyc, float *out)
{
    const uint32_t gid = blockIdx.x * 256u + threadIdx.x;
    const i32x4 a = {(int)mix(gid), (int)mix(gid + 7u), (int)mix(gid * 3u), (int)mix(gid * 5u + 1u)};
    const i32x4 b = {(int)mix(a[0]), (int)mix(a[1]), (int)mix(a[2]), (int)mix(a[3])};
    i32x4 acc[16];
    for (int q = 0; q < 16; ++q) acc[q] = i32x4{0, 0, 0, 0};
    uint32_t x[8];
    for (int q = 0; q < 8; ++q) x[q] = gid * (2u * (uint32_t)q + 3u);
    uint64_t y0 = gid, y1 = gid * 3ull;
    const uint32_t sm = __builtin_amdgcn_readfirstlane(msk);
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+a"(acc[q]) : "v"(a), "v"(b));
#pragma unroll
            for (int v = 0; v < V; ++v) {
                if constexpr (OP == 0) asm volatile("v_and_b32 %0, %1, %0" : "+v"(x[v]) : "s"(sm));
                else if constexpr (OP == 1) {
                    if (v % 2 == 0) asm volatile("v_lshlrev_b64 %0, 4, %0" : "+v"(y0));
                    else asm volatile("v_lshlrev_b64 %0, 4, %0" : "+v"(y1));
                } else asm volatile("s_nop 1");
            }
        }
    }
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    float total = (float)(y0 ^ y1);
    for (int q = 0; q < 8; ++q) total += (float)x[q];
    for (int q = 0; q < 16; ++q) total += (float)(acc[q][0] + acc[q][1] + acc[q][2] + acc[q][3]);
    out[gid] = total;
    if ((threadIdx.x & 63u) == 0) cyc[gid / 64u] = (uint32_t)(t1 - t0);
}

__device__ inline i32x4 probe_rsrc(const void *base, uint32_t n)
{
    const uint64_t p = (uint64_t)(uintptr_t)base;
    i32x4 r;
    r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)p);
    r.y = __builtin_amdgcn_readfirstlane((int)((uint32_t)(p >> 32) & 0xFFFFu));
    r.z = __builtin_amdgcn_readfirstlane((int)n);
    r.w = 0x00020000;
    return r;
}

// 5. Copies read a 2^k-byte source (plus 128 KiB of slack, which the offsets
// stay inside) as the GEMM's copies do: 8 lanes per 128-byte line, 8 rows of
// 4 KiB pitch per copy; each wave writes its own 16 KiB of the 64 KiB LDS.
// Per iteration 32 MFMAs, and BURST copies after every CPM-th; at most 40
// copies of a wave stay outstanding.  mode 1: every wave copies; 2: wave 0.
template <int CPM, int BURST>
__global__ __launch_bounds__(256) void copy_kernel(const char *src, uint32_t src_mask, int mode, int iters,
                                                   uint32_t *cyc, float *out)
{
    __shared__ __attribute__((aligned(1024))) char smem[65536];
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t gid = blockIdx.x * 256u + threadIdx.x;
    const i32x4 a = {(int)mix(gid), (int)mix(gid + 7u), (int)mix(gid * 3u), (int)mix(gid * 5u + 1u)};
    const i32x4 b = {(int)mix(a[0]), (int)mix(a[1]), (int)mix(a[2]), (int)mix(a[3])};
    i32x4 acc[16];
    for (int q = 0; q < 16; ++q) acc[q] = i32x4{0, 0, 0, 0};
    const i32x4 rs = probe_rsrc(src, src_mask + 1u + 65536u);
    const uint32_t lbase = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)smem + wave * 16384u;
    const bool copies = mode == 1 || (mode == 2 && wave == 0);
    const uint32_t lo = (lane >> 3) * 4096u + (lane & 7u) * 16u;   // < 32 KiB
    uint32_t blk = ((blockIdx.x * 4u + wave) * 32768u) & src_mask;
    uint32_t vo[16];
    for (int q = 0; q < 16; ++q) vo[q] = lo + (uint32_t)(q % 8) * 128u + (uint32_t)(q / 8) * 32768u;  // < 64 KiB
    __syncthreads();
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    // (the copying and the non-copying waves run separate loops: a branch
    // around every copy would cost more than the copy)
    if (copies) {
        for (int it = 0; it < iters; ++it) {
            int n = 0;
#pragma unroll
            for (int q = 0; q < 32; ++q) {
                asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+a"(acc[q % 16]) : "v"(a), "v"(b));
                if (q % CPM == CPM - 1) {
#pragma unroll
                    for (int c = 0; c < BURST; ++c, ++n) {
                        const uint32_t soff = __builtin_amdgcn_readfirstlane(blk);
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
                        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %3 offen lds"
                                     :
                                     : "v"(vo[n % 16]), "s"(rs), "s"(lbase + (uint32_t)(n % 16) * 1024u), "s"(soff)
                                     : "memory", "m0");
#pragma clang diagnostic pop
                    }
                }
            }
            blk = (blk + 65536u) & src_mask;
            asm volatile("s_waitcnt vmcnt(40)" ::: "memory");
        }
    } else {
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int q = 0; q < 32; ++q)
                asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+a"(acc[q % 16]) : "v"(a), "v"(b));
        }
    }
    asm volatile("s_waitcnt vmcnt(0)\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    float total = (float)smem[(threadIdx.x * 64u) & 65535u];
    for (int q = 0; q < 16; ++q) total += (float)(acc[q][0] + acc[q][1] + acc[q][2] + acc[q][3]);
    out[gid] = total;
    if (lane == 0) cyc[gid / 64u] = (uint32_t)(t1 - t0);
}

// 6. C (M x N int32) = popcount(A AND B) summed over K bits; A is M x Kw and B
// N x Kw words (row-major, K-contiguous).  A 128 x 128 tile per workgroup of
// 256 threads, each thread rows 8*ty.. and columns 8*tx.. (tx = t % 16, ty =
// t / 16).  A stage holds 16 words of K for the tile's 128 A rows and 128 B
// rows in LDS, word-major (S[w][row]) so that a thread's 8 words of one K word
// are two 16-byte reads (B: 16 threads of a wave read 128 consecutive words;
// A: broadcast).  Thread t copies row t (A for t < 128, B after) through
// registers: the next stage is loaded before the current one's arithmetic
// and written to the other LDS buffer after it.  Requires Kw % 16 == 0 (the
// host checks); rows past M or N read as zero and are not stored.
constexpr int VB_KW = 16;
__global__ __launch_bounds__(256) void valu_b1_kernel(const uint32_t *__restrict__ A, const uint32_t *__restrict__ B,
                                                      int32_t *__restrict__ C, int M, int N, int Kw, int tiles_n)
{
    __shared__ __attribute__((aligned(16))) uint32_t S[2][VB_KW][256];   // [buf][word][A rows 0..127, B rows 128..255]
    const int t = threadIdx.x, tx = t & 15, ty = t >> 4;
    const int m0 = (blockIdx.x / tiles_n) * 128, n0 = (blockIdx.x % tiles_n) * 128;
    const int row = t < 128 ? m0 + t : n0 + (t - 128);
    const bool live = t < 128 ? row < M : row < N;
    const uint32_t *src = (t < 128 ? A : B) + (int64_t)(live ? row : 0) * Kw;
    uint32_t acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0;
    uint4 st[VB_KW / 4];
    auto load = [&](int k0) {
#pragma unroll
        for (int q = 0; q < VB_KW / 4; ++q)
            st[q] = live ? *(const uint4 *)(src + k0 + 4 * q) : make_uint4(0, 0, 0, 0);
    };
    auto put = [&](int buf) {
#pragma unroll
        for (int q = 0; q < VB_KW / 4; ++q) {
            S[buf][4 * q + 0][t] = st[q].x;
            S[buf][4 * q + 1][t] = st[q].y;
            S[buf][4 * q + 2][t] = st[q].z;
            S[buf][4 * q + 3][t] = st[q].w;
        }
    };
    const int nst = Kw / VB_KW;
    load(0);
    put(0);
    __syncthreads();
    for (int s = 0; s < nst; ++s) {
        const int buf = s & 1;
        if (s + 1 < nst) load((s + 1) * VB_KW);
#pragma unroll 4
        for (int w = 0; w < VB_KW; ++w) {
            const uint4 a0 = *(const uint4 *)&S[buf][w][8 * ty], a1 = *(const uint4 *)&S[buf][w][8 * ty + 4];
            const uint4 b0 = *(const uint4 *)&S[buf][w][128 + 8 * tx], b1 = *(const uint4 *)&S[buf][w][128 + 8 * tx + 4];
            const uint32_t a[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
            const uint32_t b[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    // popcount-and-add in one instruction (as written, the
                    // compiler regroups the sums into three-input adds)
                    const uint32_t x = a[i] & b[j];
                    asm volatile("v_bcnt_u32_b32 %0, %1, %0" : "+v"(acc[i][j]) : "v"(x));
                }
        }
        if (s + 1 < nst) put(buf ^ 1);
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int m = m0 + 8 * ty + i;
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int n = n0 + 8 * tx + j;
            if (n < N) C[(int64_t)m * N + n] = (int32_t)acc[i][j];
        }
    }
}

extern "C" {

// 6. C = popcount(A AND B) GEMM on the vector ALUs (M x N, K bits with K % 512
// == 0); runs `reps` launches and returns the milliseconds between HIP events
// around them, or < 0 on a bad shape or a HIP error.
float valu_b1_run(const uint32_t *A, const uint32_t *B, int32_t *C, int M, int N, int K, int reps)
{
    if (M <= 0 || N <= 0 || K <= 0 || K % (32 * VB_KW) != 0 || reps <= 0) return -5.f;
    const int tiles_n = (N + 127) / 128;
    const int blocks = ((M + 127) / 128) * tiles_n;
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return -1.f;
    (void)hipEventRecord(e0, 0);
    for (int r = 0; r < reps; ++r)
        hipLaunchKernelGGL(valu_b1_kernel, dim3(blocks), dim3(256), 0, 0, A, B, C, M, N, K / 32, tiles_n);
    (void)hipEventRecord(e1, 0);
    if (hipEventSynchronize(e1) != hipSuccess) return -3.f;
    float ms = 0.f;
    (void)hipEventElapsedTime(&ms, e0, e1);
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    return hipGetLastError() == hipSuccess ? ms : -4.f;
}

// Launch `blocks` workgroups of slot_kernel<op, v>; cyc holds blocks * 4
// words, out blocks * 256 floats.  0 on success, < 0 on a HIP error or an
// unknown case.
int slot_run(int op, int v, int blocks, int iters, uint32_t *cyc, float *out)
{
    bool ok = false;
#define LB_PROBE_SLOT(O, N)                                                                              \
    if (!ok && op == O && v == N) {                                                                     \
        ok = true;                                                                                       \
        hipLaunchKernelGGL((slot_kernel<O, N>), dim3(blocks), dim3(256), 0, 0, iters, 0xF0F0F0F0u, cyc, out); \
    }
    LB_PROBE_SLOT(0, 0) LB_PROBE_SLOT(0, 1) LB_PROBE_SLOT(0, 2) LB_PROBE_SLOT(0, 3) LB_PROBE_SLOT(0, 4)
    LB_PROBE_SLOT(0, 8) LB_PROBE_SLOT(1, 1) LB_PROBE_SLOT(1, 2) LB_PROBE_SLOT(2, 1) LB_PROBE_SLOT(2, 2)
#undef LB_PROBE_SLOT
    if (!ok) return -5;
    return hipDeviceSynchronize() == hipSuccess && hipGetLastError() == hipSuccess ? 0 : -1;
}

// Launch `blocks` workgroups of copy_kernel<cpm, burst> over src (mask + 1 +
// 128 KiB bytes, mask + 1 a power of two); cyc holds blocks * 4 words, out
// blocks * 256 floats.  0 on success, < 0 on a HIP error or an unknown case.
int copy_run(int cpm, int burst, const char *src, uint32_t src_mask, int mode, int blocks, int iters,
             uint32_t *cyc, float *out)
{
    bool ok = false;
#define LB_PROBE_COPY(C, B)                                                                               \
    if (!ok && cpm == C && burst == B) {                                                                   \
        ok = true;                                                                                         \
        hipLaunchKernelGGL((copy_kernel<C, B>), dim3(blocks), dim3(256), 0, 0, src, src_mask, mode, iters, cyc, out); \
    }
    LB_PROBE_COPY(2, 1) LB_PROBE_COPY(4, 1) LB_PROBE_COPY(8, 1) LB_PROBE_COPY(16, 1) LB_PROBE_COPY(8, 2)
    LB_PROBE_COPY(16, 4) LB_PROBE_COPY(32, 8)
#undef LB_PROBE_COPY
    if (!ok) return -5;
    return hipDeviceSynchronize() == hipSuccess && hipGetLastError() == hipSuccess ? 0 : -1;
}

// Launch `blocks` workgroups of mix_kernel<v_per_mfma> (0..4); out holds
// blocks * 256 floats.  Milliseconds between HIP events, or < 0 on error.
float mix_rate_run(int v_per_mfma, int blocks, int iters, float *out)
{
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return -1.f;
    (void)hipEventRecord(e0, 0);
    switch (v_per_mfma) {
    case 0: hipLaunchKernelGGL(mix_kernel<0>, dim3(blocks), dim3(256), 0, 0, 99u, iters, out); break;
    case 1: hipLaunchKernelGGL(mix_kernel<1>, dim3(blocks), dim3(256), 0, 0, 99u, iters, out); break;
    case 2: hipLaunchKernelGGL(mix_kernel<2>, dim3(blocks), dim3(256), 0, 0, 99u, iters, out); break;
    case 3: hipLaunchKernelGGL(mix_kernel<3>, dim3(blocks), dim3(256), 0, 0, 99u, iters, out); break;
    case 4: hipLaunchKernelGGL(mix_kernel<4>, dim3(blocks), dim3(256), 0, 0, 99u, iters, out); break;
    default: return -2.f;
    }
    (void)hipEventRecord(e1, 0);
    if (hipEventSynchronize(e1) != hipSuccess) return -3.f;
    float ms = 0.f;
    (void)hipEventElapsedTime(&ms, e0, e1);
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    return hipGetLastError() == hipSuccess ? ms : -4.f;
}

// Launch `blocks` workgroups of store_kernel writing `chunk_bytes` each (a
// multiple of 16) into out, which must hold blocks * chunk_bytes bytes.
// Returns milliseconds between HIP events around the launch, or < 0 on error.
float store_rate_run(int blocks, int chunk_bytes, int mode, void *out)
{
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return -1.f;
    (void)hipEventRecord(e0, 0);
    hipLaunchKernelGGL(store_kernel, dim3(blocks), dim3(256), 0, 0, (i32x4 *)out, chunk_bytes / 16, mode);
    (void)hipEventRecord(e1, 0);
    if (hipEventSynchronize(e1) != hipSuccess) return -3.f;
    float ms = 0.f;
    (void)hipEventElapsedTime(&ms, e0, e1);
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    return hipGetLastError() == hipSuccess ? ms : -4.f;
}


// Launch `blocks` workgroups of 4 waves; each wave issues 16 * iters matrix
// instructions of the given kind.  out must hold blocks * 256 floats.
// Returns the elapsed milliseconds between HIP events around the launch, or a
// negative value on a HIP error.
float mfma_rate_run(int kind, int blocks, int iters, float *out)
{
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return -1.f;
    (void)hipEventRecord(e0, 0);
    switch (kind) {
    case R_I8: hipLaunchKernelGGL(rate_kernel<R_I8>, dim3(blocks), dim3(256), 0, 0, 12345u, iters, out); break;
    case R_FP8: hipLaunchKernelGGL(rate_kernel<R_FP8>, dim3(blocks), dim3(256), 0, 0, 12345u, iters, out); break;
    case R_FP6: hipLaunchKernelGGL(rate_kernel<R_FP6>, dim3(blocks), dim3(256), 0, 0, 12345u, iters, out); break;
    case R_FP4: hipLaunchKernelGGL(rate_kernel<R_FP4>, dim3(blocks), dim3(256), 0, 0, 12345u, iters, out); break;
    default: return -2.f;
    }
    (void)hipEventRecord(e1, 0);
    if (hipEventSynchronize(e1) != hipSuccess) return -3.f;
    float ms = 0.f;
    (void)hipEventElapsedTime(&ms, e0, e1);
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    return hipGetLastError() == hipSuccess ? ms : -4.f;
}

}  // extern "C"
