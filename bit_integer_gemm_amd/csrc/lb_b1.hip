// lb_b1.hip -- 1-bit GEMM on the gfx950 vector ALUs: C[m,n] = popcount over K
// of (row m of A) AND (column n of B).
//
// What is computed: the 1-bit case of the low-bit product A x B = C (digest of
// "Leveraging Large-Scale Data for Efficient Low-Bit CUTLASS GEMM Optimization
// via Neural Networks": editor's summary and the methods paragraph list 1-,
// 4- and 8-bit data; Research results item 1 gives the tiled product).  The
// product of two {0,1} elements is their AND, so 32 of them reduce with one
// v_and_b32 and one v_bcnt_u32_b32 (popcount with accumulate).
//
// How:
//  * One workgroup per BM x BN tile of C with the same multi-stage ring of
//    LDS buffers filled by direct global->LDS copies as the MFMA kernels.
//  * LDS holds each operand slice row-major (BKW words per row) in 16-byte
//    chunks whose position is XOR-swizzled by the row index, so that 16
//    consecutive rows reading the same chunk hit 16 different bank groups.
//    Each copy instruction moves whole 64..128-byte row segments, and lanes
//    pick their source chunk so that the swizzled layout comes out directly.
//  * A thread keeps a TM x TN block of int32 counts (rows ty + GY*i, columns
//    tx + GX*j) and, per 4-word chunk, reads TM + TN chunks and issues
//    TM*TN*4 AND + popcount pairs.
//  * The small tile splits each stage's K among WK waves (every wave computes
//    the whole tile on its share of K) and reduces the WK partial tiles
//    through LDS at the end, so that small problems still keep four waves per
//    workgroup busy.
#include "lb_device.hpp"
#include "lb_internal.hpp"

namespace lb {

template <int BM_, int BN_, int BKW_, int TM_, int TN_, int WK_, int ST_>
struct B1Cfg {
    static constexpr int BM = BM_, BN = BN_, BKW = BKW_, TM = TM_, TN = TN_, WK = WK_, ST = ST_;
    static constexpr int GX = BN / TN, GY = BM / TM;       // thread grid of one K group
    static constexpr int NTK = GX * GY, NT = NTK * WK, NW = NT / 64;
    static constexpr int CPR = BKW / 4;                    // 16-byte chunks per row
    static constexpr int ROWS_PER_BLK = 64 / CPR;          // rows per 1 KiB copy
    static constexpr int SWZ_DIV = 16 / CPR;               // row -> swizzle key divisor
    static constexpr int ABLK = BM / ROWS_PER_BLK, BBLK = BN / ROWS_PER_BLK;
    static constexpr int NDMA_A = ABLK / NW, NDMA_B = BBLK / NW, NDMA = NDMA_A + NDMA_B;
    static constexpr int STAGE_BYTES = (BM + BN) * BKW * 4;
    static constexpr int CH_PER_GROUP = CPR / WK;          // chunks of a stage per K group
    static constexpr int RED_BYTES = (WK - 1) * BM * BN * 4;
    static constexpr int SMEM = ST * STAGE_BYTES > RED_BYTES ? ST * STAGE_BYTES : RED_BYTES;
    static_assert(NTK % 64 == 0, "a K group is whole waves");
    static_assert(CPR >= 4 && CPR <= 16 && (CPR & (CPR - 1)) == 0, "chunks per row");
    static_assert(ABLK % NW == 0 && BBLK % NW == 0, "copies split evenly over waves");
    static_assert(CPR % WK == 0, "K groups split a stage evenly");
    static_assert(NDMA * (ST - 2) < 64, "vmcnt range");
    static_assert(SMEM <= 160 * 1024, "LDS");
};

template <class C>
__device__ inline int swz(int row) { return (row / C::SWZ_DIV) % C::CPR; }

// acc + popcount(x) as one v_bcnt_u32_b32.  Written as an instruction so that the
// compiler cannot reassociate a run of popcount additions into v_add3_u32 trees,
// which costs a third VALU op per two word pairs (measured: 1032 v_add3 next to
// 2048 v_bcnt in the medium-tile loop).
__device__ inline uint32_t popc_acc(uint32_t x, uint32_t acc)
{
    uint32_t r;
    asm("v_bcnt_u32_b32 %0, %1, %2" : "=v"(r) : "v"(x), "v"(acc));
    return r;
}

// Byte offset in a stage of chunk c of local row r (A rows first, then B rows).
template <class C>
__device__ inline int chunk_off(int r, int c) { return (r * C::CPR + (c ^ swz<C>(r))) * 16; }

template <class C>
__device__ inline void b1_zero_k_tail(char *stage, uint32_t lane, uint32_t wave, int64_t kw0,
                                      int64_t Kw)
{
#pragma unroll
    for (int i = 0; i < C::NDMA_A; ++i) {
        const int j = (int)wave + C::NW * i;
        const int row = j * C::ROWS_PER_BLK + (int)lane / C::CPR;
        const int c = ((int)lane % C::CPR) ^ swz<C>(row);
        if (kw0 + 4 * c >= Kw)
            *(u32x4 *)(stage + j * 1024 + lane * 16) = u32x4{0, 0, 0, 0};
    }
}

template <int N, int ST>
__device__ inline void b1_wait(int tiles_after)
{
    if constexpr (ST == 2) {
        wait_vm_barrier<0>();
    } else if constexpr (ST == 3) {
        if (tiles_after >= 1) wait_vm_barrier<N>(); else wait_vm_barrier<0>();
    } else {
        if (tiles_after >= 2) wait_vm_barrier<2 * N>();
        else if (tiles_after == 1) wait_vm_barrier<N>();
        else wait_vm_barrier<0>();
    }
}

template <class C>
__global__ __launch_bounds__(C::NT) void b1_gemm_kernel(
    const uint32_t *__restrict__ A, const uint32_t *__restrict__ B, int32_t *__restrict__ Cout,
    int32_t M, int32_t N, int32_t Kw, uint32_t tiles_m, uint32_t tiles_n)
{
    __shared__ __attribute__((aligned(1024))) char smem[C::SMEM];

    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = (int)(tid / C::NTK);           // K group
    const int t = (int)(tid % C::NTK);
    const int tx = t % C::GX, ty = t / C::GX;

    uint32_t tm, tn;
    tile_of_block(blockIdx.x, tiles_m, tiles_n, 8u, tm, tn);
    const int64_t m0 = (int64_t)tm * C::BM, n0 = (int64_t)tn * C::BN;
    const int64_t rowbytes = (int64_t)Kw * 4;
    const uint32_t *Ab = A + m0 * Kw;
    const uint32_t *Bb = B + n0 * Kw;
    const int64_t a_bytes = (int64_t)(M - m0) * rowbytes;
    const int64_t b_bytes = (int64_t)(N - n0) * rowbytes;

    uint32_t voff[C::NDMA];
#pragma unroll
    for (int i = 0; i < C::NDMA; ++i) {
        const bool isA = i < C::NDMA_A;
        const int j = (int)wave + C::NW * (isA ? i : i - C::NDMA_A);
        const int row = j * C::ROWS_PER_BLK + (int)lane / C::CPR;   // row inside A or B slice
        const int c = ((int)lane % C::CPR) ^ swz<C>(isA ? row : C::BM + row);
        voff[i] = (uint32_t)(row * rowbytes + c * 16);
    }
    const uint32_t smem_base = lds_addr(smem);

    auto issue = [&](int64_t kt, int slot) {
        const int64_t kbyte = kt * C::BKW * 4;
        const i32x4 ra = make_rsrc((const char *)Ab + kbyte, a_bytes > kbyte ? (uint64_t)(a_bytes - kbyte) : 0);
        const i32x4 rb = make_rsrc((const char *)Bb + kbyte, b_bytes > kbyte ? (uint64_t)(b_bytes - kbyte) : 0);
        const uint32_t sbase = smem_base + slot * C::STAGE_BYTES;
#pragma unroll
        for (int i = 0; i < C::NDMA; ++i) {
            const bool isA = i < C::NDMA_A;
            const int j = (int)wave + C::NW * (isA ? i : i - C::NDMA_A);
            dma16(isA ? ra : rb, voff[i], sbase + (isA ? j : C::ABLK + j) * 1024);
        }
    };

    uint32_t acc[C::TM][C::TN];
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j) acc[i][j] = 0;

    const int64_t nk = ((int64_t)Kw + C::BKW - 1) / C::BKW;
    const bool k_tail = (Kw % C::BKW) != 0;

#pragma unroll
    for (int s = 0; s < C::ST - 1; ++s)
        if (s < nk) issue(s, s);

    for (int64_t kt = 0; kt < nk; ++kt) {
        const int slot = (int)(kt % C::ST);
        const int64_t after = nk - 1 - kt;
        b1_wait<C::NDMA, C::ST>((int)(after < C::ST - 2 ? after : C::ST - 2));
        char *stage = smem + slot * C::STAGE_BYTES;
        if (k_tail && kt == nk - 1) {
            b1_zero_k_tail<C>(stage, lane, wave, kt * C::BKW, Kw);
            barrier_lds();
        }
        if (kt + C::ST - 1 < nk) issue(kt + C::ST - 1, (int)((kt + C::ST - 1) % C::ST));

#pragma unroll
        for (int cc = 0; cc < C::CH_PER_GROUP; ++cc) {
            const int c = grp * C::CH_PER_GROUP + cc;
            u32x4 a[C::TM], b[C::TN];
#pragma unroll
            for (int i = 0; i < C::TM; ++i)
                a[i] = *(const u32x4 *)(stage + chunk_off<C>(ty + C::GY * i, c));
#pragma unroll
            for (int j = 0; j < C::TN; ++j)
                b[j] = *(const u32x4 *)(stage + chunk_off<C>(C::BM + tx + C::GX * j, c));
#pragma unroll
            for (int w = 0; w < 4; ++w)
#pragma unroll
                for (int i = 0; i < C::TM; ++i)
#pragma unroll
                    for (int j = 0; j < C::TN; ++j)
                        acc[i][j] = popc_acc(a[i][w] & b[j][w], acc[i][j]);
        }
    }

    if constexpr (C::WK > 1) {
        // Reduce the K groups' partial tiles through LDS (the stage ring is free now).
        barrier_lds();
        uint32_t *red = (uint32_t *)smem;
        if (grp > 0) {
#pragma unroll
            for (int i = 0; i < C::TM; ++i)
#pragma unroll
                for (int j = 0; j < C::TN; ++j)
                    red[((grp - 1) * C::BM + ty + C::GY * i) * C::BN + tx + C::GX * j] = acc[i][j];
        }
        barrier_lds();
        if (grp != 0) return;
#pragma unroll
        for (int g = 1; g < C::WK; ++g)
#pragma unroll
            for (int i = 0; i < C::TM; ++i)
#pragma unroll
                for (int j = 0; j < C::TN; ++j)
                    acc[i][j] += red[((g - 1) * C::BM + ty + C::GY * i) * C::BN + tx + C::GX * j];
    }

#pragma unroll
    for (int i = 0; i < C::TM; ++i) {
        const int64_t m = m0 + ty + C::GY * i;
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < C::TN; ++j) {
            const int64_t n = n0 + tx + C::GX * j;
            if (n < N) Cout[m * (int64_t)N + n] = (int32_t)acc[i][j];
        }
    }
}

// index = 3*tile + (stages - 2)
using BS2 = B1Cfg<64, 64, 32, 8, 8, 4, 2>;
using BS3 = B1Cfg<64, 64, 32, 8, 8, 4, 3>;
using BS4 = B1Cfg<64, 64, 32, 8, 8, 4, 4>;
using BM2 = B1Cfg<128, 128, 32, 8, 8, 1, 2>;
using BM3 = B1Cfg<128, 128, 32, 8, 8, 1, 3>;
using BM4 = B1Cfg<128, 128, 32, 8, 8, 1, 4>;
using BL2 = B1Cfg<256, 128, 16, 8, 8, 1, 2>;
using BL3 = B1Cfg<256, 128, 16, 8, 8, 1, 3>;
using BL4 = B1Cfg<256, 128, 16, 8, 8, 1, 4>;

template <class C>
static hipError_t b1_launch_one(const uint32_t *A, const uint32_t *B, int32_t *Cout, int64_t M,
                                int64_t N, int64_t Kw, hipStream_t s)
{
    const uint64_t tm = (uint64_t)((M + C::BM - 1) / C::BM);
    const uint64_t tn = (uint64_t)((N + C::BN - 1) / C::BN);
    if (tm * tn > 0x7FFFFFFFull) return hipErrorInvalidValue;
    hipLaunchKernelGGL((b1_gemm_kernel<C>), dim3((uint32_t)(tm * tn)), dim3(C::NT), 0, s, A, B, Cout,
                       (int32_t)M, (int32_t)N, (int32_t)Kw, (uint32_t)tm, (uint32_t)tn);
    return hipGetLastError();
}

template <class C>
static void b1_info_one(int *bm, int *bn, int *bk, int *st)
{
    *bm = C::BM; *bn = C::BN; *bk = C::BKW; *st = C::ST;
}

hipError_t launch_b1(int variant, const uint32_t *A, const uint32_t *B, int32_t *Cout, int64_t M,
                     int64_t N, int64_t Kw, hipStream_t s)
{
    switch (variant) {
    case 0: return b1_launch_one<BS2>(A, B, Cout, M, N, Kw, s);
    case 1: return b1_launch_one<BS3>(A, B, Cout, M, N, Kw, s);
    case 2: return b1_launch_one<BS4>(A, B, Cout, M, N, Kw, s);
    case 3: return b1_launch_one<BM2>(A, B, Cout, M, N, Kw, s);
    case 4: return b1_launch_one<BM3>(A, B, Cout, M, N, Kw, s);
    case 5: return b1_launch_one<BM4>(A, B, Cout, M, N, Kw, s);
    case 6: return b1_launch_one<BL2>(A, B, Cout, M, N, Kw, s);
    case 7: return b1_launch_one<BL3>(A, B, Cout, M, N, Kw, s);
    case 8: return b1_launch_one<BL4>(A, B, Cout, M, N, Kw, s);
    default: return hipErrorInvalidValue;
    }
}

int b1_variant_info(int variant, int *bm, int *bn, int *bk_words, int *stages)
{
    switch (variant) {
    case 0: b1_info_one<BS2>(bm, bn, bk_words, stages); return 0;
    case 1: b1_info_one<BS3>(bm, bn, bk_words, stages); return 0;
    case 2: b1_info_one<BS4>(bm, bn, bk_words, stages); return 0;
    case 3: b1_info_one<BM2>(bm, bn, bk_words, stages); return 0;
    case 4: b1_info_one<BM3>(bm, bn, bk_words, stages); return 0;
    case 5: b1_info_one<BM4>(bm, bn, bk_words, stages); return 0;
    case 6: b1_info_one<BL2>(bm, bn, bk_words, stages); return 0;
    case 7: b1_info_one<BL3>(bm, bn, bk_words, stages); return 0;
    case 8: b1_info_one<BL4>(bm, bn, bk_words, stages); return 0;
    default: return -1;
    }
}

}  // namespace lb
