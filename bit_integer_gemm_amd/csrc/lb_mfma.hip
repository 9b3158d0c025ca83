// lb_mfma.hip -- int8 / int4 / 1-bit GEMM, the int8 linear layer and the
// low-bit convolution on gfx950 int8 MFMA.
//
// What is computed: C = A x B with exact int32 accumulation for 8-bit and
// 4-bit operands (digest of "Leveraging Large-Scale Data for Efficient Low-Bit
// CUTLASS GEMM Optimization via Neural Networks": editor's summary for the bit
// widths, Research results item 1 for the tiled product), and the linear layer
// of Research results item 4 with a per-row x per-column fp32 dequantisation
// fused into the store.
//
// How (MI355X-first; the pages' CUTLASS/Tensor-Core design is prior art):
//  * One workgroup per BM x BN tile of C, NW waves in a WM x WN grid; each wave
//    owns a (BM/WM) x (BN/WN) sub-tile held in int32 accumulators.
//  * K is walked in stages of BK bytes.  A stage is an LDS buffer holding the
//    A and B slices as 1 KiB blocks of 16 rows x 64 K-bytes.  One copy
//    instruction fills one block: lanes 4r..4r+3 fetch the four 16-byte
//    chunks of row r (one contiguous 64-byte segment, so the address
//    coalescer merges them; spreading consecutive lanes over 16 rows instead
//    cuts delivered bandwidth by 2-3x), and the chunk order inside each row
//    is XOR-permuted by (r/2)%4.  The MFMA fragment read (lane i takes row
//    i%16, chunk i/16) is then free of LDS bank conflicts: ds_read_b128 is
//    served 8 lanes at a time, and rows r..r+7 with the same chunk land in 8
//    distinct 16-byte bank groups (measured: 0 SQ_LDS_BANK_CONFLICT, while a
//    (r/4)%4 permutation or none costs ~20% of LDS read throughput).
//  * ST stages (2, 3 or 4) form a ring filled by direct global->LDS copies
//    issued ST-1 stages ahead (the multi-stage pipeline of Research results
//    item 1; the 2-stage case is classic double buffering).
//  * v_mfma_i32_16x16x64_i8 with the B fragment as the first source and the A
//    fragment as the second: the 4 accumulators of lane i then hold
//    C[m = i%16][n = 4*(i/16) .. +3], four consecutive columns, so the store is
//    one 16-byte write per lane.  Any permutation of K shared by A and B leaves
//    the product unchanged, so the MFMA's internal K order need not match
//    memory order.
//  * int4: the LDS holds packed bytes.  After the LDS read each 32-bit word w
//    becomes lo = (w << 4) & 0xF0F0F0F0 (even k) and hi = w & 0xF0F0F0F0 (odd
//    k): every nibble moves to the top of its own byte, i.e. the int8 value
//    16*v with v's sign bit as the byte's sign bit.  MFMA then sums 256*a*b
//    exactly and an arithmetic shift by 8 recovers C.
//  * 1-bit: the LDS holds packed bits, 64 bytes = 512 values of K per block
//    row, and a fragment read gives each lane 16 bytes (128 bits) of its row.
//    MFMA step s (0..7) takes bit s of each of those 16 bytes, and the int8
//    MFMA sums the products exactly, eight steps per 64-byte block.  The AND
//    of two bits is their product, so this is the same popcount(a AND b) sum,
//    at the matrix cores' rate instead of the vector ALUs'.  Byte j of step s
//    is K index 128*(lane/16) + 8*j + s of the block for A and B alike, a
//    permutation of K that both operands share.  To need one AND per operand
//    and step, A's bytes are bit-mirrored and shifted down one place once per
//    fragment (bit s -> bit 6-s); step s < 7 keeps A's bit as 2^(6-s) and B's
//    as 2^s, so every pair of set bits adds 64 (bit 7: 64 and 1), and the
//    epilogue divides by 64.
//  * Rows past M or N read as zero through the buffer range check; a partial
//    last K stage has its out-of-range A pieces zeroed in LDS before use.
//  * A launch may cover a band of C: the output's row stride is an argument
//    (a band of columns), and a grid with several rows of workgroups splits K
//    (row y sums bytes [y*ksplit, (y+1)*ksplit) of K and adds its exact
//    partial sums into a zeroed C with atomic adds; integer GEMMs only).
//  * Convolution (the im2win convolution summary, gist.science paper
//    2608.20725, method: NHWC images, a window per output) runs through the
//    same kernel: row r of A is output pixel r and its K axis walks the filter
//    taps (kh, kw) and the channels.  The page's window tensor is never built:
//    each copy lane reads its 16-byte piece of the window straight from the
//    NHWC image, the window tensor's addressing without its memory.  Channel
//    bytes per pixel are a multiple of 16, so every 16-byte piece sits inside
//    a single tap (when they are a multiple of 64, a whole 64-byte K block
//    does, and the tap is the block's); pieces that fall in the zero padding
//    (or past M or K) get an offset with bit 31 set, beyond the buffer range,
//    and load zero.
#include <algorithm>
#include <type_traits>

#include "lb_device.hpp"
#include "lb_internal.hpp"

namespace lb {

template <int BM_, int BN_, int BK_, int WM_, int WN_, int ST_>
struct MfmaCfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_, ST = ST_;
    static constexpr int NW = WM * WN, NT = NW * 64;
    static constexpr int TM = BM / WM, TN = BN / WN;  // wave sub-tile
    static constexpr int FM = TM / 16, FN = TN / 16;  // 16x16 fragments per wave
    static constexpr int KB = BK / 64;                // 64-byte K blocks per stage
    static constexpr int ABLK = (BM / 16) * KB, BBLK = (BN / 16) * KB;
    static constexpr int NDMA_A = ABLK / NW, NDMA_B = BBLK / NW, NDMA = NDMA_A + NDMA_B;
    static constexpr int STAGE_BYTES = (ABLK + BBLK) * 1024;
    static_assert(BK % 64 == 0 && TM % 16 == 0 && TN % 16 == 0, "tile shape");
    static_assert(ABLK % NW == 0 && BBLK % NW == 0, "copies must split evenly over waves");
    static_assert(NDMA * (ST - 2) < 64, "vmcnt range");
    static_assert(ST * STAGE_BYTES <= 160 * 1024, "LDS");
};

// Design choices that profiling builds can turn off, one at a time, for A/B
// measurements (the library is always built with the defaults; the package's
// build tool makes the A/B libraries, see its --ab option):
//   LB_AB_LDS_SWIZZLE=0     no XOR permutation of 16-byte chunks in LDS
//                           (fragment reads then collide on LDS banks)
//   LB_AB_COPY_ROWS_SPREAD=1 in the 16-row blocks, consecutive copy lanes take
//                           16 different rows instead of 4 lanes per row
//   LB_AB_TILE_MAP_PLAIN=1  workgroups take tiles in row-major order (no XCD
//                           runs, no bands)
//   LB_AB_COPY_BURST=1      four-wave int8 tile: a refill's 16 copies per
//                           wave all go out in the odd block's second half,
//                           one per two MFMAs (instead of one per four over
//                           that half and the next block's first half)
//   LB_AB_W4_INT8_ONLY=1    int4 and 1-bit large 2-stage variant on the 8-wave
//                           tile of the general kernel instead of the
//                           four-wave tile
//   LB_AB_W4_BANDS=1        four-wave tile: XCD runs and bands of tile rows for
//                           every grid width (not row-major order when the
//                           width is a multiple of 64 tiles)
//   LB_AB_REG_STAGING=1     general kernel: operand stages go global ->
//                           registers -> LDS (a buffer load into registers
//                           when the stage is issued, written to LDS at the
//                           start of the next K step) instead of the direct
//                           global -> LDS copy; the prologue writes each stage
//                           at once
// Each keeps the results exact; only the speed changes.
#ifndef LB_AB_LDS_SWIZZLE
#define LB_AB_LDS_SWIZZLE 1
#endif
#ifndef LB_AB_COPY_ROWS_SPREAD
#define LB_AB_COPY_ROWS_SPREAD 0
#endif
#ifndef LB_AB_COPY_BURST
#define LB_AB_COPY_BURST 0
#endif
#ifndef LB_AB_W4_INT8_ONLY
#define LB_AB_W4_INT8_ONLY 0
#endif
#ifndef LB_AB_W4_BANDS
#define LB_AB_W4_BANDS 0
#endif
#ifndef LB_AB_REG_STAGING
#define LB_AB_REG_STAGING 0
#endif

// Layout of a 16-row x 64-byte block: row r's chunk c sits at 16-byte slot
// 4*r + (c ^ ((r >> 1) & 3)).  A copy lane i fills slot i, i.e. row i/4.
// (A/B build with spread copies: slot 16*c + r, lane i takes row i%16, chunk
// i/16, and the fragment read of lane l is slot l.)
__device__ inline uint32_t blk_row_of_lane(uint32_t lane)
{
    return LB_AB_COPY_ROWS_SPREAD ? lane & 15u : lane >> 2;
}
__device__ inline uint32_t blk_chunk_of_lane(uint32_t lane)
{
    if (LB_AB_COPY_ROWS_SPREAD) return lane >> 4;
    return LB_AB_LDS_SWIZZLE ? (lane & 3u) ^ ((lane >> 3) & 3u) : lane & 3u;
}
__device__ inline uint32_t frag_offset(uint32_t lane)
{
    if (LB_AB_COPY_ROWS_SPREAD) return lane * 16u;
    const uint32_t r = lane & 15u, c = lane >> 4;
    return (4u * r + (LB_AB_LDS_SWIZZLE ? c ^ ((r >> 1) & 3u) : c)) * 16u;
}

// Out-of-range K pieces of A in the last (partial) stage are zeroed in LDS:
// with A's extra K at zero, whatever B holds there contributes nothing.
template <class C>
__device__ inline void zero_k_tail(char *stage, uint32_t lane, uint32_t wave,
                                   int64_t k0, int64_t Kb)
{
#pragma unroll
    for (int i = 0; i < C::NDMA_A; ++i) {
        const int j = (int)wave + C::NW * i;
        const int kb = j / (C::BM / 16);
        const int64_t kbyte = k0 + kb * 64 + (int)blk_chunk_of_lane(lane) * 16;
        if (kbyte >= Kb)
            *(i32x4 *)(stage + j * 1024 + lane * 16) = i32x4{0, 0, 0, 0};
    }
}

template <int N, int ST>
__device__ inline void wait_outstanding(int tiles_after)
{
    // tiles_after = number of later stages already in flight (0..ST-2)
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

__device__ inline i32x4 mfma16(i32x4 a, i32x4 b, i32x4 c)
{
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// int4 even-k plane of a packed fragment: (w << 4) & 0xF0F0F0F0 per word.  The
// shifts go two words at a time as 64-bit shifts; the bits that cross from one
// word into the next land in a low nibble, which the mask clears.  The unpack
// is on the int4 loop's critical path (its vector instructions overlap the
// MFMAs little): two 64-bit shifts instead of four 32-bit ones made every int4
// variant 1.3-3.4% faster (4096^3, large 2-stage tile: 52.5 against 53.7 us).
// The compiler turns a 64-bit shift of a 64-bit value into two 32-bit
// instructions here, hence the one-instruction assembly.
__device__ inline i32x4 s4_even_plane(i32x4 w)
{
    uint64_t p0 = ((uint64_t)(uint32_t)w.y << 32) | (uint32_t)w.x;
    uint64_t p1 = ((uint64_t)(uint32_t)w.w << 32) | (uint32_t)w.z;
    asm("v_lshlrev_b64 %0, 4, %1" : "=v"(p0) : "v"(p0));
    asm("v_lshlrev_b64 %0, 4, %1" : "=v"(p1) : "v"(p1));
    i32x4 r;
    r.x = (int32_t)((uint32_t)p0 & 0xF0F0F0F0u);
    r.y = (int32_t)((uint32_t)(p0 >> 32) & 0xF0F0F0F0u);
    r.z = (int32_t)((uint32_t)p1 & 0xF0F0F0F0u);
    r.w = (int32_t)((uint32_t)(p1 >> 32) & 0xF0F0F0F0u);
    return r;
}

// Bits of each byte in reverse order, then the whole word shifted down one
// place: bit s (s < 7) of every byte lands on bit 6 - s of the same byte (bit 7
// of each byte then holds a bit of the next byte, which no mask below keeps).
__device__ inline i32x4 mirror_bytes_shr1(i32x4 w)
{
    u32x4 u = (u32x4)w;
#pragma unroll
    for (int d = 0; d < 4; ++d) u[d] = __builtin_bswap32(__builtin_bitreverse32(u[d])) >> 1;
    return (i32x4)u;
}

// 1-bit route on the FP4 matrix instruction (v_mfma_scale_f32_16x16x128_f8f6f4
// with e2m1 operands on both sides).  Plane s (0..3) of a lane's 16 bytes keeps
// bit 4j+s of every word in nibble j, the rest of the nibble zero: 32 e2m1
// values per lane, each 0 or 2^(s-1) (nibble codes 0001 = 0.5, 0010 = 1.0,
// 0100 = 2.0).  Bit 3 of a nibble is the e2m1 sign bit (0.0 or -0.0 alone), so
// plane 3 is shifted down one place and takes the code 0100 = 2.0.  A and B
// get the same planes, so the product of two set bits is 4^(s-1) (planes 0-2)
// or 4 (plane 3), and the E8M0 block scales 2^(1-s) (2^-1 for plane 3) on each
// operand bring every such product to exactly 1.0.  The fp32 accumulator then
// holds the count exactly while it stays below 2^24.  One instruction covers
// 128 K bits of a 16x16 tile, twice the int8 route's 64.
template <int S>
__device__ inline i32x4 fp4_plane(i32x4 w)
{
    const u32x4 u = (u32x4)w;
    if constexpr (S < 3) return (i32x4)(u & (0x11111111u << S));
    else return (i32x4)((u >> 1) & 0x44444444u);
}
template <int S>
__device__ inline f32x4 mfma_fp4(i32x4 b, i32x4 a, f32x4 c)
{
    typedef int i32x8 __attribute__((ext_vector_type(8)));
    constexpr int sc = S == 0 ? 128 : S == 1 ? 127 : 126;  // E8M0: 2^(sc - 127)
    const i32x8 b8 = {b.x, b.y, b.z, b.w, 0, 0, 0, 0}, a8 = {a.x, a.y, a.z, a.w, 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b8, a8, c, 4, 4, 0, sc, 0, sc);
}

template <class C, int KIND, bool CONV>
__global__ __launch_bounds__(C::NT) void mfma_gemm_kernel(
    const int8_t *__restrict__ A, const int8_t *__restrict__ B, void *__restrict__ out,
    const float *__restrict__ sx, const float *__restrict__ sw,
    int32_t M, int32_t N, int32_t Kb, uint32_t tiles_m, uint32_t tiles_n, int32_t ldo,
    int32_t ksplit, ConvGeom g)
{
    // Linear layer: the tile's row and column scales follow the stage ring
    // (medium and large tiles; the small tile keeps its five workgroups per CU
    // and reads the scales from global memory).
    constexpr bool LDS_SCALES = KIND == KIND_LINEAR && C::BM >= 128;
    // LATE_COPIES (four-wave tiles and int4): the next stage's copies go out
    // right after the stage wait, ahead of this stage's fragment reads; the
    // other tiles issue them behind the first fragment reads (see the loop).
    constexpr bool LATE_COPIES = C::NW == 4 || KIND == KIND_S4;
    constexpr int SCALE_BYTES = LDS_SCALES ? (C::BM + C::BN) * 4 : 0;
    __shared__ __attribute__((aligned(1024))) char smem[C::ST * C::STAGE_BYTES + SCALE_BYTES];

    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t wm = wave / C::WN, wn = wave % C::WN;

    // Bands of 4 tile rows for the medium and large tiles, 8 for the small
    // one (see tile_of_block).  Measured per variant against 8-row bands, one
    // build each in one process: the default large tile 4.6-5% faster (int8
    // 4096^3, 8192 x 8192 x 4096), the 3-stage medium tile 4.5-6.5% (int8 K =
    // 1024 at 8192^2 and 16384^2), the 1-bit large tile 1.6-4.5%, the 2-stage
    // medium tile within 0.5%; the small tile 8% slower at 2048^3.
    uint32_t tm, tn;
    tile_of_block(blockIdx.x, tiles_m, tiles_n, C::BM >= 128 ? 4u : 8u, tm, tn);
    const int64_t m0 = (int64_t)tm * C::BM, n0 = (int64_t)tn * C::BN;

    // Split K: workgroup row blockIdx.y sums K bytes [kbeg, kbeg + klen) of the
    // product and adds its partial result into C (which the host zeroed); a
    // grid of one row covers all of K (ksplit = Kb) and stores.  Kb stays the
    // row stride of A and B.
    const int64_t kbeg = (int64_t)blockIdx.y * ksplit;
    const int32_t klen = (int32_t)((int64_t)Kb - kbeg < ksplit ? (int64_t)Kb - kbeg : (int64_t)ksplit);
    const bool accumulate = gridDim.y > 1;
    const int8_t *Ab = A + m0 * Kb + kbeg;
    const int8_t *Bb = B + n0 * Kb + kbeg;
    const int64_t a_bytes = (int64_t)(M - m0) * Kb - kbeg;
    const int64_t b_bytes = (int64_t)(N - n0) * Kb - kbeg;

    // Per-copy lane offsets inside the tile (constant over K).
    uint32_t voff[C::NDMA];
#pragma unroll
    for (int i = 0; i < C::NDMA; ++i) {
        const bool isA = i < C::NDMA_A;
        const int j = (int)wave + C::NW * (isA ? i : i - C::NDMA_A);
        const int rows = isA ? C::BM / 16 : C::BN / 16;
        const int rb = j % rows, kb = j / rows;
        // 32-bit offsets: at most 255 rows of Kb bytes, below 2^32 for every
        // accepted K (unsigned arithmetic, so long rows wrap nothing).
        voff[i] = (uint32_t)(rb * 16 + (int)blk_row_of_lane(lane)) * (uint32_t)Kb +
                  (uint32_t)(kb * 64 + (int)blk_chunk_of_lane(lane) * 16);
    }
    const uint32_t smem_base = lds_addr(smem);

    // Convolution: per A copy, the window origin of its output pixel and the
    // byte offset of that origin's channel piece (valid only inside the image).
    int32_t cv_hi0[C::NDMA_A], cv_wi0[C::NDMA_A], cv_base[C::NDMA_A];
    bool cv_row[C::NDMA_A];
    int32_t cv_kh = 0, cv_kw = 0, cv_cb = 0;  // first K block of the next stage to copy
    if constexpr (CONV) {
        const int32_t hw = g.Ho * g.Wo;
#pragma unroll
        for (int i = 0; i < C::NDMA_A; ++i) {
            const int j = (int)wave + C::NW * i;
            const int32_t r = (int32_t)m0 + (j % (C::BM / 16)) * 16 + (int32_t)blk_row_of_lane(lane);
            cv_row[i] = r < M;
            const int32_t rr = cv_row[i] ? r : 0;
            const int32_t n = rr / hw, rem = rr - n * hw;
            const int32_t ho = rem / g.Wo, wo = rem - ho * g.Wo;
            cv_hi0[i] = ho * g.sh - g.ph;
            cv_wi0[i] = wo * g.sw - g.pw;
            cv_base[i] = ((n * g.H + cv_hi0[i]) * g.W + cv_wi0[i]) * g.Cb +
                         (int32_t)blk_chunk_of_lane(lane) * 16;
        }
    }
    // Advance a (kh, kw, channel byte) position by one 64-byte K block: one tap
    // when Cb is a multiple of 64, else as many taps as the block crosses
    // (Cb a multiple of 16: at most four).
    auto next_block = [&](int32_t &kh, int32_t &kw, int32_t &cb) {
        cb += 64;
        while (cb >= g.Cb) {
            cb -= g.Cb;
            if (++kw >= g.Kw) { kw = 0; ++kh; }
        }
    };

    // (A/B build with register staging: the stage issued last, held in
    // registers until commit() writes it to its LDS slot.)
    i32x4 stg[LB_AB_REG_STAGING ? C::NDMA : 1];
    int stg_slot = -1;
    auto issue = [&](int64_t kt, int slot) {
        const int64_t k0 = kt * C::BK;
        i32x4 ra;
        if constexpr (CONV) ra = make_rsrc(A, g.x_bytes);
        else ra = make_rsrc(Ab + k0, a_bytes > k0 ? (uint64_t)(a_bytes - k0) : 0);
        const i32x4 rb = make_rsrc(Bb + k0, b_bytes > k0 ? (uint64_t)(b_bytes - k0) : 0);
        // Filter tap and channel byte of each K block of this stage (stages are
        // copied in order, one call per stage).
        int32_t bkh[C::KB], bkw[C::KB], bcb[C::KB];
        if constexpr (CONV) {
#pragma unroll
            for (int b = 0; b < C::KB; ++b) {
                bkh[b] = cv_kh; bkw[b] = cv_kw; bcb[b] = cv_cb;
                next_block(cv_kh, cv_kw, cv_cb);
            }
        }
        const uint32_t sbase = smem_base + slot * C::STAGE_BYTES;
#pragma unroll
        for (int i = 0; i < C::NDMA; ++i) {
            const bool isA = i < C::NDMA_A;
            const int j = (int)wave + C::NW * (isA ? i : i - C::NDMA_A);
            const uint32_t dst = sbase + (isA ? j : C::ABLK + j) * 1024;
            uint32_t vo = voff[i];
            if constexpr (CONV) {
                if (isA) {
                    const int kb = j / (C::BM / 16);
                    int32_t kh = bkh[0], kw = bkw[0], cb = bcb[0];
#pragma unroll
                    for (int b = 1; b < C::KB; ++b)
                        if (kb == b) { kh = bkh[b]; kw = bkw[b]; cb = bcb[b]; }
                    int32_t base = cv_base[i];
                    if (g.Cb % 64 != 0) {
                        // Fewer than 64 bytes per tap (or not a multiple): this
                        // lane's 16-byte chunk lies chunk*16 bytes past the
                        // block's first byte, up to three taps further on.
                        const int32_t ch = (int32_t)blk_chunk_of_lane(lane) * 16;
                        base -= ch;
                        cb += ch;
#pragma unroll
                        for (int w = 0; w < 3; ++w)
                            if (cb >= g.Cb) {
                                cb -= g.Cb;
                                if (++kw >= g.Kw) { kw = 0; ++kh; }
                            }
                    }
                    const int32_t hi = cv_hi0[i] + kh, wi = cv_wi0[i] + kw;
                    const bool ok = cv_row[i] && kh < g.Kh && (uint32_t)hi < (uint32_t)g.H &&
                                    (uint32_t)wi < (uint32_t)g.W;
                    vo = ok ? (uint32_t)(base + (kh * g.W + kw) * g.Cb + cb) : 0x80000000u;
                }
            }
            if constexpr (LB_AB_REG_STAGING) stg[i] = load16(isA ? ra : rb, vo);
            else dma16(isA ? ra : rb, vo, dst);
        }
        if constexpr (LB_AB_REG_STAGING) stg_slot = slot;
    };
    auto commit = [&]() {
        if constexpr (LB_AB_REG_STAGING) {
            if (stg_slot >= 0) {
                char *sb = smem + stg_slot * C::STAGE_BYTES;
#pragma unroll
                for (int i = 0; i < C::NDMA; ++i) {
                    const bool isA = i < C::NDMA_A;
                    const int j = (int)wave + C::NW * (isA ? i : i - C::NDMA_A);
                    *(i32x4 *)(sb + (isA ? j : C::ABLK + j) * 1024 + lane * 16) = stg[i];
                }
                stg_slot = -1;
            }
        }
    };

    using Acc = std::conditional_t<KIND == KIND_B1F4, f32x4, i32x4>;
    Acc acc[C::FM][C::FN];
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) acc[i][j] = Acc{0, 0, 0, 0};

    const int64_t nk = ((int64_t)klen + C::BK - 1) / C::BK;
    const bool k_tail = (klen % C::BK) != 0;

    // Linear layer: wave 0 copies sx[m0 .. m0+BM) and sw[n0 .. n0+BN) into LDS
    // ahead of the first stage (entries past M or N read as zero).  These copies
    // are older than every stage copy, so the first stage wait covers them, and
    // the epilogue reads the scales from LDS instead of waiting on global loads
    // at the end of the tile (5% of the layer's time at 8192 x 11008 x 4096).
    if constexpr (LDS_SCALES) {
        if (wave == 0) {
            const uint32_t sbase = smem_base + C::ST * C::STAGE_BYTES;
            const i32x4 rx = make_rsrc(sx + m0, (uint64_t)(M - m0) * 4);
            const i32x4 rw = make_rsrc(sw + n0, (uint64_t)(N - n0) * 4);
#pragma unroll
            for (int q = 0; q < C::BM / 64; ++q) dma4(rx, lane * 4 + q * 256, sbase + q * 256);
#pragma unroll
            for (int q = 0; q < C::BN / 64; ++q) dma4(rw, lane * 4 + q * 256, sbase + C::BM * 4 + q * 256);
        }
    }
#pragma unroll
    for (int s = 0; s < C::ST - 1; ++s)
        if (s < nk) {
            issue(s, s);
            commit();
        }

    for (int64_t kt = 0; kt < nk; ++kt) {
        const int slot = (int)(kt % C::ST);
        const int64_t after = nk - 1 - kt;
        if constexpr (LB_AB_REG_STAGING) {
            commit();
            barrier_lds();
        } else {
            wait_outstanding<C::NDMA, C::ST>((int)(after < C::ST - 2 ? after : C::ST - 2));
        }
        char *stage = smem + slot * C::STAGE_BYTES;
        if (k_tail && kt == nk - 1) {
            zero_k_tail<C>(stage, lane, wave, kt * C::BK, klen);
            barrier_lds();
        }
        if constexpr (LATE_COPIES)
            if (kt + C::ST - 1 < nk) issue(kt + C::ST - 1, (int)((kt + C::ST - 1) % C::ST));

        const char *fstage = stage + frag_offset(lane);
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb) {
            i32x4 af[C::FM], bf[C::FN];
#pragma unroll
            for (int i = 0; i < C::FM; ++i)
                af[i] = *(const i32x4 *)(fstage + (kb * (C::BM / 16) + wm * C::FM + i) * 1024);
#pragma unroll
            for (int j = 0; j < C::FN; ++j)
                bf[j] = *(const i32x4 *)(fstage + (C::ABLK + kb * (C::BN / 16) + wn * C::FN + j) * 1024);
            // Large tiles: the next stage's copies go out behind this stage's
            // first fragment reads (they fill the slot the previous iteration
            // read, which the barrier above has released), so the LDS latency
            // of the reads runs under the copies' address arithmetic; the MFMAs
            // stay below them.  Measured: 1-2% faster for the large int8 and
            // 1-bit tiles, 5% slower for the small tile.  The int4 tiles copy
            // first: holding their fragments over the copies would spill.
            if (kb == 0) {
                if constexpr (!LATE_COPIES) {
                    if (kt + C::ST - 1 < nk) issue(kt + C::ST - 1, (int)((kt + C::ST - 1) % C::ST));
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            if constexpr (KIND == KIND_S4) {
                i32x4 alo[C::FM], ahi[C::FM];
#pragma unroll
                for (int i = 0; i < C::FM; ++i) {
                    alo[i] = s4_even_plane(af[i]);
                    ahi[i] = af[i] & (int)0xF0F0F0F0;
                }
#pragma unroll
                for (int j = 0; j < C::FN; ++j) {
                    const i32x4 blo = s4_even_plane(bf[j]);
                    const i32x4 bhi = bf[j] & (int)0xF0F0F0F0;
#pragma unroll
                    for (int i = 0; i < C::FM; ++i) {
                        acc[i][j] = mfma16(blo, alo[i], acc[i][j]);
                        acc[i][j] = mfma16(bhi, ahi[i], acc[i][j]);
                    }
                }
            } else if constexpr (KIND == KIND_B1) {
                // Bit 7 of every byte first, from the words as loaded: A's as
                // the value 64, B's as the value 1.
                {
                    i32x4 ea[C::FM];
#pragma unroll
                    for (int i = 0; i < C::FM; ++i) ea[i] = (i32x4)(((u32x4)af[i] >> 1) & 0x40404040u);
#pragma unroll
                    for (int j = 0; j < C::FN; ++j) {
                        const i32x4 eb = (i32x4)(((u32x4)bf[j] >> 7) & 0x01010101u);
#pragma unroll
                        for (int i = 0; i < C::FM; ++i) acc[i][j] = mfma16(eb, ea[i], acc[i][j]);
                    }
                }
                // Bits 0..6: A's byte bit s moves to bit 6-s, so one AND per
                // operand gives A's bit s as 2^(6-s) and B's as 2^s.
#pragma unroll
                for (int i = 0; i < C::FM; ++i) af[i] = mirror_bytes_shr1(af[i]);
                auto step = [&](auto sc) {
                    constexpr int st = decltype(sc)::value;
                    i32x4 ea[C::FM];
#pragma unroll
                    for (int i = 0; i < C::FM; ++i) ea[i] = (i32x4)((u32x4)af[i] & (0x01010101u << (6 - st)));
#pragma unroll
                    for (int j = 0; j < C::FN; ++j) {
                        const i32x4 eb = (i32x4)((u32x4)bf[j] & (0x01010101u << st));
#pragma unroll
                        for (int i = 0; i < C::FM; ++i) acc[i][j] = mfma16(eb, ea[i], acc[i][j]);
                    }
                };
                step(std::integral_constant<int, 0>{});
                step(std::integral_constant<int, 1>{});
                step(std::integral_constant<int, 2>{});
                step(std::integral_constant<int, 3>{});
                step(std::integral_constant<int, 4>{});
                step(std::integral_constant<int, 5>{});
                step(std::integral_constant<int, 6>{});
            } else if constexpr (KIND == KIND_B1F4) {
                auto plane = [&](auto sc) {
                    constexpr int st = decltype(sc)::value;
                    i32x4 ea[C::FM];
#pragma unroll
                    for (int i = 0; i < C::FM; ++i) ea[i] = fp4_plane<st>(af[i]);
#pragma unroll
                    for (int j = 0; j < C::FN; ++j) {
                        const i32x4 eb = fp4_plane<st>(bf[j]);
#pragma unroll
                        for (int i = 0; i < C::FM; ++i) acc[i][j] = mfma_fp4<st>(eb, ea[i], acc[i][j]);
                    }
                };
                plane(std::integral_constant<int, 0>{});
                plane(std::integral_constant<int, 1>{});
                plane(std::integral_constant<int, 2>{});
                plane(std::integral_constant<int, 3>{});
            } else {
#pragma unroll
                for (int i = 0; i < C::FM; ++i)
#pragma unroll
                    for (int j = 0; j < C::FN; ++j) acc[i][j] = mfma16(bf[j], af[i], acc[i][j]);
            }
        }
    }

    // Epilogue: lane holds C[m][n..n+3] for each fragment.
    const bool vec_ok = ((N | ldo) & 3) == 0;
    const float *lds_sx = (const float *)(smem + C::ST * C::STAGE_BYTES);
    const float *lds_sw = lds_sx + C::BM;
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
        const int64_t m = m0 + wm * C::TM + i * 16 + (lane % 16);
        if (m >= M) continue;
        float scale_m = 0.f;
        if constexpr (KIND == KIND_LINEAR) scale_m = LDS_SCALES ? lds_sx[m - m0] : sx[m];
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
            const int64_t n = n0 + wn * C::TN + j * 16 + (lane / 16) * 4;
            if (n >= N) continue;
            i32x4 v;
            if constexpr (KIND == KIND_B1F4) {
                // exact: the fp32 sums are integers below 2^24
                v = i32x4{(int32_t)acc[i][j].x, (int32_t)acc[i][j].y, (int32_t)acc[i][j].z,
                          (int32_t)acc[i][j].w};
            } else {
                v = acc[i][j];
            }
            if constexpr (KIND == KIND_S4) v = v >> 8;
            if constexpr (KIND == KIND_B1) v = v >> 6;
            if constexpr (KIND == KIND_LINEAR) {
                float *o = (float *)out + m * (int64_t)ldo + n;
                if (vec_ok) {
                    const f32x4 s = LDS_SCALES ? *(const f32x4 *)(lds_sw + (n - n0))
                                               : *(const f32x4 *)(sw + n);
                    f32x4 r;
                    r.x = ((float)v.x * scale_m) * s.x;
                    r.y = ((float)v.y * scale_m) * s.y;
                    r.z = ((float)v.z * scale_m) * s.z;
                    r.w = ((float)v.w * scale_m) * s.w;
                    *(f32x4 *)o = r;
                } else {
                    for (int r = 0; r < 4 && n + r < N; ++r) o[r] = ((float)v[r] * scale_m) * (LDS_SCALES ? lds_sw[n - n0 + r] : sw[n + r]);
                }
            } else {
                int32_t *o = (int32_t *)out + m * (int64_t)ldo + n;
                if (accumulate) {
                    for (int r = 0; r < 4 && n + r < N; ++r) atomicAdd(o + r, v[r]);
                } else if (vec_ok) {
                    *(i32x4 *)o = v;
                } else {
                    for (int r = 0; r < 4 && n + r < N; ++r) o[r] = v[r];
                }
            }
        }
    }
}

// ---- large tile on four waves (int8, int4, 1-bit, int8 linear) ----------
// The 2-stage large variant of the int8, int4 and 1-bit (FP4 route) GEMMs and
// of the int8 linear layer: a 256x256 tile on four waves (one per SIMD) of
// 128x128, all 256 accumulators of a lane in AGPRs.  Per workgroup, per 64
// K-bytes: 64 KiB of LDS fragment reads for 256 MFMAs (int4: 512; 1-bit: 1024
// FP4 MFMAs), against 128 KiB for sixteen waves of 64x64.
//  * Two LDS super-stages of 128 K-bytes (64 KiB each: 256 A rows, 256 B rows)
//    form the 2-stage ring.  A 2 KiB block holds 16 rows x 128 bytes as two
//    1 KiB halves of 8 rows; row r's 16-byte chunk c sits at
//    (r/8)*1024 + (r%8)*128 + 16*(c ^ (r%8)).  One copy fills one half: lane
//    i reads chunk (i%8) ^ (i/8) of row i/8, so each 8 lanes read one whole
//    128-byte line.  The fragment read of K half h (lane l: row l%16, chunk
//    l/16 + 4h) is conflict-free: the 8 lanes served together hold rows
//    r..r+7 of one half, at distinct slots (c + 4h) ^ (r%8).
//  * Block t (64 K-bytes) is half t%2 of super-stage t/2.  Each block runs
//    its MFMAs in two halves (rows 0-3, then 4-7 of the wave's 8x8 fragment
//    grid); the next block's 16 fragments (B first: the next block's first
//    row needs all of them) are read between the second half's MFMAs, so LDS
//    latency stays under the matrix cores.  After the first half of an odd
//    block every wave is done with that block's super-stage: wait for the
//    next super-stage's copies, barrier, and refill the free slot with the
//    super-stage after next (the pipeline of Research results item 1, two
//    stages deep).
//  * The refill's 16 copies per wave go out one per four MFMA slots: copies
//    0-7 between the second half's MFMAs, 8-15 between those of the next
//    (even) block's first half, which still leaves one block of MFMAs before
//    the wait.  A copy costs its wave about 11-14 cycles next to the MFMAs, but
//    a CU's copy path moves 64 bytes per cycle: the earlier schedule, four
//    waves each issuing 16 copies within 32 MFMAs, saturated it and stalled
//    every wave (cycle counts at int8 4096^3: 97.0k loop cycles per wave
//    against 70.3k for the MFMAs alone; spread, 87.6k).  When no super-stage
//    is left to load, the copies read an empty buffer range (zeros, no memory
//    traffic) into the slot just released, which nothing reads again, so the
//    copy code has no branches (a branch per copy cost several percent).
//  * int4 and 1-bit: the LDS holds packed bytes, and each fragment is turned
//    in registers into the planes the MFMAs take (int4: even-k and odd-k
//    nibbles, two MFMAs per fragment pair; 1-bit: four FP4 bit planes, four
//    MFMAs).  With one wave per SIMD nothing else hides that vector work, so
//    it is written as single-instruction asm statements placed between the
//    MFMAs (measured: up to two vector instructions per MFMA issue free, each
//    further one costs about 4 cycles), each plane complete at least two
//    instructions before the MFMA that reads it.  Every copy serves two
//    (int4) or four (1-bit) times the MFMAs of the int8 tile.
//  * The MFMA is inline assembly with the accumulator tied to its AGPR: with
//    the builtin the compiler picks the untied form and shuffles all 256
//    accumulators between register files.  Its operands come straight from
//    LDS reads (the compiler waits for them); the accumulators are read only
//    after 32 wait states past the last MFMA.
__device__ inline uint32_t wide_chunk_of_lane(uint32_t lane)
{
    return LB_AB_LDS_SWIZZLE ? (lane & 7u) ^ (lane >> 3) : lane & 7u;
}
__device__ inline uint32_t wide_frag_offset(uint32_t lane, uint32_t h)
{
    const uint32_t r = lane & 15u, c = (lane >> 4) + 4u * h;
    return (r >> 3) * 1024u + (r & 7u) * 128u + 16u * (LB_AB_LDS_SWIZZLE ? c ^ (r & 7u) : c);
}
__device__ inline void mfma_tied(i32x4 &c, i32x4 a, i32x4 b)
{
    asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}

// Item of a spread schedule at MFMA slot s: H items over S slots (S >= H),
// item c at slot floor(c*S/H) (OFF = 0) or floor((c+1)*S/H) - 1 (OFF = 1);
// -1 if no item falls on s.
template <int S, int H, int OFF>
__device__ constexpr int spread_item(int s)
{
    for (int c = 0; c < H; ++c)
        if (((c + OFF) * S) / H - OFF == s) return c;
    return -1;
}

// FM x FN: fragment rows and columns of a wave's sub-tile (16 x 16 each); the
// workgroup tile is (32*FM) x (32*FN).  8 x 8 (256x256) serves every type;
// 8 x 6 (256x192) serves every type, 6 x 8 (192x256) the int8 GEMM and the
// linear layer, when a product's 256x256
// tiles would fill less than one round of the CUs (the host picks them for an
// automatic choice).  The copies and the next
// block's fragment reads are spread over a half-block's MFMA slots by
// spread_item; for 8 x 8 that is the fixed pattern of one copy per four slots
// and one read per two.
template <int KIND, int FM, int FN>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void mfma_w4_kernel(
    const int8_t *__restrict__ A, const int8_t *__restrict__ B, void *__restrict__ out,
    const float *__restrict__ sx, const float *__restrict__ sw,
    int32_t M, int32_t N, int32_t Kb, uint32_t tiles_m, uint32_t tiles_n, int32_t ldo, int32_t ksplit)
{
    static_assert(FM % 2 == 0 && FM >= 4 && FM <= 8 && FN % 2 == 0 && FN >= 4 && FN <= 8, "wave sub-tile");
    static_assert((FM == 8 && FN == 8) || KIND == KIND_S8 || KIND == KIND_LINEAR ||
                      ((KIND == KIND_S4 || KIND == KIND_B1F4) && FM == 8 && FN == 6),
                  "int4 and 1-bit run the 256x256 and 256x192 tiles");
    constexpr int BM = 32 * FM, BN = 32 * FN;
    constexpr int SS = (BM + BN) * 128;   // one super-stage: 128 K-bytes of A and B
    constexpr int BOFF = BM * 128;        // B's blocks within a super-stage
    constexpr int NCP = FM + FN;          // refill copies per wave per super-stage
    constexpr int SCALE_BYTES = KIND == KIND_LINEAR ? (BM + BN) * 4 : 0;
    __shared__ __attribute__((aligned(1024))) char smem[2 * SS + SCALE_BYTES];
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t wm = wave >> 1, wn = wave & 1u;
    // A grid 64 tiles wide (or a multiple) takes tiles in row-major order:
    // round robin over the XCDs then gives each XCD every eighth column of
    // the same rows.  Same-machine interleaved timings against the XCD runs with
    // bands of 4 rows, int8: 4096 x 16384 x 4096 243.1 against 270.0 us,
    // 16384^2 x 4096 961 against 1058 us; 32 tiles wide it was mixed (8192^2 x
    // 4096 251.4 against 260.8 us, but 2048 x 8192 x 4096 60.8 against 58.3 us
    // and int4 16384 x 8192 x 8192 715 against 701 us); 16 wide equal within
    // 1% (4096^3, where it read 50% more bytes past L2), 48 wide 0.6% slower,
    // 43 wide (the linear layer) 2.7% slower.  Other grids keep the XCD runs
    // and bands of 4 tile rows: against 8, int8 8192 x 8192 x 4096 241.6
    // against 283.9 us and 16384 x 4096 x 4096 233.6 against 236.7 us, 4096^3
    // equal (bands of 2: 239.6, 267.2, 59.1 us).
    uint32_t tm, tn;
    if (tiles_n % 64u == 0u && !LB_AB_W4_BANDS) {
        tm = blockIdx.x / tiles_n;
        tn = blockIdx.x % tiles_n;
    } else {
        tile_of_block(blockIdx.x, tiles_m, tiles_n, 4u, tm, tn);
    }
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

    // Split K as in the other kernels: row blockIdx.y of the grid sums K bytes
    // [kbeg, kbeg + klen) and adds its partial sums into a zeroed C.
    const int64_t kbeg = (int64_t)blockIdx.y * ksplit;
    const int32_t klen = (int32_t)((int64_t)Kb - kbeg < ksplit ? (int64_t)Kb - kbeg : (int64_t)ksplit);
    const bool accumulate = gridDim.y > 1;
    const int8_t *Ab = A + m0 * Kb + kbeg;
    const int8_t *Bb = B + n0 * Kb + kbeg;
    const int64_t a_bytes = (int64_t)(M - m0) * Kb - kbeg;
    const int64_t b_bytes = (int64_t)(N - n0) * Kb - kbeg;

    // Copy q (0..FM-1 for A, 0..FN-1 for B) of wave w fills half u%2 of block
    // u/2, u = w + 4q.
    constexpr int NV = FM > FN ? FM : FN;
    uint32_t voff[NV];
#pragma unroll
    for (int q = 0; q < NV; ++q) {
        const int u = (int)wave + 4 * q;
        voff[q] = (uint32_t)((u / 2) * 16 + (u % 2) * 8 + (int)(lane >> 3)) * (uint32_t)Kb +
                  wide_chunk_of_lane(lane) * 16u;
    }
    const uint32_t smem_base = lds_addr(smem);
    auto rsrc_a = [&](int ss) {
        const int64_t k0 = (int64_t)ss * 128;
        return make_rsrc(Ab + k0, a_bytes > k0 ? (uint64_t)(a_bytes - k0) : 0);
    };
    auto rsrc_b = [&](int ss) {
        const int64_t k0 = (int64_t)ss * 128;
        return make_rsrc(Bb + k0, b_bytes > k0 ? (uint64_t)(b_bytes - k0) : 0);
    };
    auto copy_q = [&](const i32x4 &ra, const i32x4 &rb, uint32_t sbase, int q) {
        if (q < FM) dma16(ra, voff[q], sbase + ((int)wave + 4 * q) * 1024);
        else dma16(rb, voff[q - FM], sbase + BOFF + ((int)wave + 4 * (q - FM)) * 1024);
    };
    // A pieces past the band's K are zeroed once their super-stage has landed.
    auto zero_tail = [&](int slot, int64_t k0) {
#pragma unroll
        for (int q = 0; q < FM; ++q) {
            const int u = (int)wave + 4 * q;
            if (k0 + (int)wide_chunk_of_lane(lane) * 16 >= klen)
                *(i32x4 *)(smem + slot * SS + u * 1024 + lane * 16) = i32x4{0, 0, 0, 0};
        }
    };

    // (1-bit, FP4 route: the accumulators hold fp32 bits, exact counts; a
    // zero word is 0.0.)
    i32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = i32x4{0, 0, 0, 0};

    const int nss = (klen + 127) / 128;  // super-stages
    const int nk = (klen + 63) / 64;     // 64-byte blocks
    const bool k_tail = (klen % 128) != 0;
    // Linear layer: wave 0 copies sx[m0 .. m0+BM) and sw[n0 .. n0+BN) into LDS
    // before the first super-stage (entries past M or N read as zero); the first
    // stage wait covers these older copies, and the epilogue reads the scales
    // from LDS (read from global memory at the end of the tile, they made the
    // layer 5% slower at 8192 x 11008 x 4096).
    if constexpr (KIND == KIND_LINEAR) {
        if (wave == 0) {
            const uint32_t sbase = smem_base + 2 * SS;
            const i32x4 rx = make_rsrc(sx + m0, (uint64_t)(M - m0) * 4);
            const i32x4 rw = make_rsrc(sw + n0, (uint64_t)(N - n0) * 4);
#pragma unroll
            for (int q = 0; q < BM / 64; ++q) dma4(rx, lane * 4 + q * 256, sbase + q * 256);
#pragma unroll
            for (int q = 0; q < BN / 64; ++q) dma4(rw, lane * 4 + q * 256, sbase + BM * 4 + q * 256);
        }
    }
    {
        const i32x4 ra = rsrc_a(0), rb = rsrc_b(0);
#pragma unroll
        for (int q = 0; q < NCP; ++q) copy_q(ra, rb, smem_base, q);
    }
    if (nss > 1) {
        const i32x4 ra = rsrc_a(1), rb = rsrc_b(1);
#pragma unroll
        for (int q = 0; q < NCP; ++q) copy_q(ra, rb, smem_base + SS, q);
        wait_vm_barrier<NCP>();
    } else {
        wait_vm_barrier<0>();
    }
    if (k_tail && nss == 1) {
        zero_tail(0, 0);
        barrier_lds();
    }
    const uint32_t foff0 = wide_frag_offset(lane, 0), foff1 = wide_frag_offset(lane, 1);
    auto fptr = [&](int t) { return smem + ((t / 2) % 2) * SS + ((t % 2) ? foff1 : foff0); };
    // int4: the offsets are remade per block from the lane (a few vector
    // instructions) rather than held across the loop in two registers.
    auto fptr4 = [&](int t) {
        uint32_t l = lane;
        asm volatile("" : "+v"(l));
        return smem + ((t / 2) % 2) * SS + wide_frag_offset(l, (uint32_t)(t % 2));
    };

    i32x4 fa0[FM], fb0[FN], fa1[FM], fb1[FN];
    {
        const char *f = fptr(0);
#pragma unroll
        for (int i = 0; i < FM; ++i) fa0[i] = *(const i32x4 *)(f + (wm * FM + i) * 2048);
#pragma unroll
        for (int j = 0; j < FN; ++j) fb0[j] = *(const i32x4 *)(f + BOFF + (wn * FN + j) * 2048);
    }

    // Refill of the slot released at the last odd block's barrier (no refill
    // due: an empty buffer range, read into that slot).  Before the first
    // barrier there is none, and the first block issues no copies.
    const i32x4 none = make_rsrc(A, 0);
    i32x4 cra = none, crb = none;
    uint32_t csb = smem_base;
    auto copy_r = [&](int q) { copy_q(cra, crb, csb, q); };

    // MFMAs of fragment rows i0 .. i0+FM/2-1 (int8).  CP: issue refill copies,
    // NCP/2 spread evenly over the half's FM/2 x FN MFMA slots: copies
    // NCP/2.. in an even block's first half, 0..NCP/2-1 in an odd block's
    // second half (8 x 8: one per four slots).  The second half also reads
    // the next block's FM + FN fragments from f, B first, spread likewise
    // (8 x 8: one per two slots).
    auto half = [&](auto cp_c, const i32x4 *fa, const i32x4 *fb, int i0, bool second, const char *f,
                    i32x4 *na, i32x4 *nb) {
        constexpr bool CP = decltype(cp_c)::value;
        constexpr int S = FM / 2 * FN, H = NCP / 2;
#pragma unroll
        for (int i = i0; i < i0 + FM / 2; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int sl = (i - i0) * FN + j;
                mfma_tied(acc[i][j], fb[j], fa[i]);
                if (LB_AB_COPY_BURST) {
                    const int c = spread_item<S, NCP, 0>(sl);
                    if (CP && second && c >= 0) copy_r(c);
                } else if (CP) {
                    const int c = spread_item<S, H, 0>(sl);
                    if (c >= 0) copy_r((second ? 0 : H) + c);
                }
                if (second) {
                    const int q = spread_item<S, FM + FN, 1>(sl);
                    if (q >= 0 && q < FN) nb[q] = *(const i32x4 *)(f + BOFF + (wn * FN + q) * 2048);
                    else if (q >= FN) na[q - FN] = *(const i32x4 *)(f + (wm * FM + q - FN) * 2048);
                }
            }
    };
    // One 64-byte K block; PAR = t % 2, FIRST: block 0 (no refill pending).
    auto body = [&](auto par_c, auto first_c, int t, const i32x4 *ca, const i32x4 *cb, i32x4 *na,
                    i32x4 *nb) {
        constexpr int PAR = decltype(par_c)::value;
        constexpr bool FIRST = decltype(first_c)::value;
        half(std::integral_constant<bool, PAR == 0 && !FIRST && !LB_AB_COPY_BURST>{}, ca, cb, 0, false, nullptr, na, nb);
        if constexpr (PAR == 1) {
            wait_vm_barrier<0>();
            const int ss = t / 2;
            const bool more = ss + 2 < nss;
            cra = more ? rsrc_a(ss + 2) : none;
            crb = more ? rsrc_b(ss + 2) : none;
            csb = smem_base + (uint32_t)((ss % 2) * SS);
            if (k_tail && ss + 1 == nss - 1) {
                zero_tail((ss + 1) % 2, (int64_t)(nss - 1) * 128);
                barrier_lds();
            }
        }
        // After the last block the reads fetch stale LDS that nothing uses.
        half(std::integral_constant<bool, PAR == 1>{}, ca, cb, FM / 2, true, fptr(t + 1), na, nb);
    };
    // int4 and 1-bit: refill copies walk their offsets (copy q of a wave reads
    // 32 rows of K bytes past copy q-1) in one register instead of eight.
    const uint32_t kstride = (uint32_t)Kb * 32u;
    uint32_t vcur = voff[0];
    auto copy_r4 = [&](int q) {
        if (q % 8 == 0) vcur = voff[0];
        dma16(q < 8 ? cra : crb, vcur,
              csb + (q < 8 ? 0u : (uint32_t)BOFF) + ((uint32_t)wave + 4u * (uint32_t)(q % 8)) * 1024u);
        asm volatile("v_add_u32 %0, %1, %0" : "+v"(vcur) : "s"(kstride));
    };
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    using F0 = std::false_type;
    if constexpr (KIND == KIND_S8 || KIND == KIND_LINEAR) {
        body(P0{}, std::true_type{}, 0, fa0, fb0, fa1, fb1);
        int t = 1;
        for (; t + 1 < nk; t += 2) {
            body(P1{}, F0{}, t, fa1, fb1, fa0, fb0);
            body(P0{}, F0{}, t + 1, fa0, fb0, fa1, fb1);
        }
        if (t < nk) body(P1{}, F0{}, t, fa1, fb1, fa0, fb0);
    } else if constexpr (KIND == KIND_S4) {
        // int4.  Per block (128 MFMA slots per wave) 160 vector instructions
        // make the even-k and odd-k planes of 16 fragments.  Next to a wave's
        // own MFMAs about two vector instructions per MFMA issue free, and
        // each further one costs about 4 cycles (measured), so they are
        // placed one by one: each is an asm statement, kept in order with the
        // MFMAs.  A planes, one register set: the next row's even-k plane is
        // made in slots 8-13 of a row (after its last even-k MFMA), a row's
        // odd-k plane in its slots 0-3.  B fragments of the next block: read
        // in the first eight slots of the second half into the odd-k plane
        // array and unpacked in place, their 80 instructions spread over the
        // half's slots 12-63 (at most two per slot); the B planes are double
        // buffered.  A fragments of the next block: read in the second half
        // over the ones whose planes are made (single buffer).  Every plane is
        // complete at least two instructions before its first MFMA (the
        // hazard the compiler does not check around assembly MFMAs).
        i32x4 *fa = fa0;
        i32x4 *bhi4[2] = {fb0, fb1};   // packed B, then its odd-k plane in place
        i32x4 blo4[2][FN];             // even-k planes of B
        const int msk = __builtin_amdgcn_readfirstlane((int)0xF0F0F0F0);
        auto shl4 = [](int lo, int hi) {
            uint64_t x = ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
            asm volatile("v_lshlrev_b64 %0, 4, %1" : "=v"(x) : "v"(x));
            return x;
        };
        auto andm = [&](int x) {
            int r;
            asm volatile("v_and_b32 %0, %1, %2" : "=v"(r) : "s"(msk), "v"(x));
            return r;
        };
        // Step k (0..9) of making planes (lo, hi) of packed fragment w: the
        // 64-bit shifts write lo's register pairs, which are then masked in
        // place; hi may be w itself (in place).
        auto plane_op = [&](int k, i32x4 &w, i32x4 &lo, i32x4 &hi) {
            if (k == 0 || k == 1) {
                const uint64_t x = shl4(k == 0 ? w.x : w.z, k == 0 ? w.y : w.w);
                if (k == 0) { lo.x = (int)(uint32_t)x; lo.y = (int)(uint32_t)(x >> 32); }
                else { lo.z = (int)(uint32_t)x; lo.w = (int)(uint32_t)(x >> 32); }
            }
            else if (k == 2) lo.x = andm(lo.x);
            else if (k == 3) lo.y = andm(lo.y);
            else if (k == 4) lo.z = andm(lo.z);
            else if (k == 5) lo.w = andm(lo.w);
            else if (k == 6) hi.x = andm(w.x);
            else if (k == 7) hi.y = andm(w.y);
            else if (k == 8) hi.z = andm(w.z);
            else hi.w = andm(w.w);
        };
        i32x4 alo, ahi;
        // Block 0: its B planes and row 0's A planes before the first MFMA.
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int k = 0; k < 10; ++k) plane_op(k, bhi4[0][j], blo4[0][j], bhi4[0][j]);
#pragma unroll
        for (int k = 0; k < 10; ++k) plane_op(k, fa[0], alo, ahi);
        asm volatile("s_nop 1" ::: "memory");

        auto body4 = [&](auto par_c, auto first_c, int t) {
            constexpr int P = decltype(par_c)::value, Q = 1 - P;
            constexpr bool FIRST = decltype(first_c)::value;
            const char *f = fptr4(t + 1);
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const bool second = i >= FM / 2;
                if (i == FM / 2 && P == 1) {
                    wait_vm_barrier<0>();
                    const int ss = t / 2;
                    const bool more = ss + 2 < nss;
                    cra = more ? rsrc_a(ss + 2) : none;
                    crb = more ? rsrc_b(ss + 2) : none;
                    csb = smem_base + (uint32_t)((ss % 2) * SS);
                    if (k_tail && ss + 1 == nss - 1) {
                        zero_tail((ss + 1) % 2, (int64_t)(nss - 1) * 128);
                        barrier_lds();
                    }
                }
#pragma unroll
                for (int sl = 0; sl < 2 * FN; ++sl) {
                    const int j = sl % FN;
                    const bool odd = sl >= FN;
                    mfma_tied(acc[i][j], odd ? bhi4[P][j] : blo4[P][j], odd ? ahi : alo);
                    // refill copies: 8-15 in an even block's first half, 0-7 in an
                    // odd block's second half, two per row
                    // (256x192: the six B copies in rows 0-2 of the even block)
                    const bool cp = second ? P == 1 : (P == 0 && !FIRST);
                    if constexpr (FN == 8) {
                        if (cp && sl % FN == 0) copy_r4((second ? 0 : 8) + (i % (FM / 2)) * 2 + sl / FN);
                    } else {
                        const int cq = (second ? 0 : 8) + (i % (FM / 2)) * 2 + sl / FN;
                        if (cp && sl % FN == 0 && cq < FM + FN) copy_r4(cq);
                    }
                    const int z = (i - FM / 2) * 2 * FN + sl;  // slot in the second half
                    if (second && z < FN) bhi4[Q][z] = *(const i32x4 *)(f + BOFF + (wn * FN + z) * 2048);
                    // the next block's A fragment q replaces fragment q once
                    // this block's planes of row q are made: q <= 4 in row 4,
                    // later ones in their own row, at slots 8-12
                    if (second && sl >= FN && sl < FN + 5) {
                        const int q = i == FM / 2 ? sl - FN : (sl == FN ? i : -1);
                        if (q >= 0) fa[q] = *(const i32x4 *)(f + (wm * FM + q) * 2048);
                    }
                    // A planes: the next row's even-k plane into alo after this
                    // row's last even-k MFMA (slots 8-13; after row FM-1 the next
                    // block's row 0), this row's odd-k plane into ahi in slots 0-3
                    // (this row's first odd-k MFMA is at slot 8).  With six
                    // fragment columns (12 slots a row) the even-k plane takes two
                    // instructions a slot in slots 6-8, so that it is complete
                    // three MFMAs before the next row's first.
                    if constexpr (FN == 8) {
                        if (sl >= FN && sl < FN + 6) plane_op(sl - FN, fa[(i + 1) % FM], alo, ahi);
                    } else if (sl >= FN && sl < FN + 3) {
                        plane_op(2 * (sl - FN), fa[(i + 1) % FM], alo, ahi);
                        plane_op(2 * (sl - FN) + 1, fa[(i + 1) % FM], alo, ahi);
                    }
                    if (sl < 4) plane_op(6 + sl, fa[i], alo, ahi);
                    // the next block's B planes: instruction u of 10 FN at
                    // second-half slot 12 + u (S2 - 12) / (10 FN), S2 the half's
                    // slots (8 x 8: 12 + 52u/80)
                    if (second && z >= 12) {
                        constexpr int S2 = FM / 2 * 2 * FN;
#pragma unroll
                        for (int u = 0; u < 10 * FN; ++u)
                            if (12 + (u * (S2 - 12)) / (10 * FN) == z)
                                plane_op(u % 10, bhi4[Q][u / 10], blo4[Q][u / 10], bhi4[Q][u / 10]);
                    }
                }
            }
        };
        body4(P0{}, std::true_type{}, 0);
        int t = 1;
        for (; t + 1 < nk; t += 2) {
            body4(P1{}, F0{}, t);
            body4(P0{}, F0{}, t + 1);
        }
        if (t < nk) body4(P1{}, F0{}, t);
    } else {
        // 1-bit on the FP4 instruction.  A block's 64 K-bytes are 512 bits per
        // row, four planes of 128 (see fp4_plane): 256 MFMAs per wave, taken
        // plane by plane (32 rows (plane p, fragment row i) of 8), so that one
        // plane of B (8 fragments, 32 registers) is live at a time and the
        // two MFMAs into one accumulator are 64 apart.  The planes are made one
        // step ahead by single vector instructions placed between the MFMAs
        // (about two per MFMA issue free next to a wave's own MFMAs): in row
        // (p, i) the A plane of the next row and B plane p+1 of fragment i.
        // Packed fragments are single-buffered: in plane 3, once this block's
        // last planes are made, the next block's B fragments are read in row
        // (3, 0) and its A fragment i in row (3, i), and the next block's
        // plane-0 planes are made from them in rows (3, 1..7).  Every plane is
        // complete at least two instructions before its first MFMA.
        i32x4 *fa = fa0, *fb = fb0;
        i32x4 bp[2][FN];   // B planes p (even p) and p+1 (odd p): double buffer
        i32x4 ap[2];       // A planes of the current and the next row
        const int m0s = __builtin_amdgcn_readfirstlane(0x11111111), m1s = __builtin_amdgcn_readfirstlane(0x22222222),
                  m2s = __builtin_amdgcn_readfirstlane(0x44444444);
        // E8M0 block scales per plane: 2^(1-s), plane 3 2^-1 (its nibbles hold 2.0)
        int sc0 = 128, sc1 = 127, sc2 = 126;
        asm volatile("" : "+v"(sc0), "+v"(sc1), "+v"(sc2));
        auto andm = [](int x, int m) {
            int r;
            asm volatile("v_and_b32 %0, %1, %2" : "=v"(r) : "s"(m), "v"(x));
            return r;
        };
        auto shr1 = [](int lo, int hi) {
            uint64_t x = ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
            asm volatile("v_lshrrev_b64 %0, 1, %1" : "=v"(x) : "v"(x));
            return x;
        };
        auto nops = [](int p) { return p == 3 ? 6 : 4; };
        // Step k of making plane p of packed fragment w into x.
        auto plane_op = [&](int p, int k, const i32x4 &w, i32x4 &x) {
            if (p < 3) {
                const int m = p == 0 ? m0s : p == 1 ? m1s : m2s;
                if (k == 0) x.x = andm(w.x, m);
                else if (k == 1) x.y = andm(w.y, m);
                else if (k == 2) x.z = andm(w.z, m);
                else x.w = andm(w.w, m);
            } else if (k == 0 || k == 1) {
                const uint64_t v = shr1(k == 0 ? w.x : w.z, k == 0 ? w.y : w.w);
                if (k == 0) { x.x = (int)(uint32_t)v; x.y = (int)(uint32_t)(v >> 32); }
                else { x.z = (int)(uint32_t)v; x.w = (int)(uint32_t)(v >> 32); }
            }
            else if (k == 2) x.x = andm(x.x, m2s);
            else if (k == 3) x.y = andm(x.y, m2s);
            else if (k == 4) x.z = andm(x.z, m2s);
            else x.w = andm(x.w, m2s);
        };
        auto mfma_b1 = [&](i32x4 &c, const i32x4 &b, const i32x4 &a, int s) {
            asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %3 op_sel_hi:[0,0,0] cbsz:4 blgp:4"
                         : "+a"(c) : "v"(b), "v"(a), "v"(s));
        };
        // Block 0: B plane 0 and row (0, 0)'s A plane before the first MFMA.
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int k = 0; k < 4; ++k) plane_op(0, k, fb[j], bp[0][j]);
#pragma unroll
        for (int k = 0; k < 4; ++k) plane_op(0, k, fa[0], ap[0]);
        asm volatile("s_nop 1" ::: "memory");

        // Half H of a block (planes 2H and 2H+1, 128 MFMAs; unrolled as one
        // piece the whole block outgrows the compiler's unrolling).
        auto half1 = [&](auto par_c, auto first_c, auto half_c, int t) {
            constexpr int P = decltype(par_c)::value, H = decltype(half_c)::value;
            constexpr bool FIRST = decltype(first_c)::value;
            const char *f = fptr4(t + 1);
            if (H == 1 && P == 1) {
                wait_vm_barrier<0>();
                const int ss = t / 2;
                const bool more = ss + 2 < nss;
                cra = more ? rsrc_a(ss + 2) : none;
                crb = more ? rsrc_b(ss + 2) : none;
                csb = smem_base + (uint32_t)((ss % 2) * SS);
                if (k_tail && ss + 1 == nss - 1) {
                    zero_tail((ss + 1) % 2, (int64_t)(nss - 1) * 128);
                    barrier_lds();
                }
            }
#pragma unroll
            for (int p = 2 * H; p < 2 * H + 2; ++p)
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int r = p * FM + i;
                // the next row (after row (3, 7): the next block's row (0, 0))
                const int pn = (r + 1) / FM % 4, in = (r + 1) % FM;
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    mfma_b1(acc[i][j], bp[p % 2][j], ap[r % 2], p == 0 ? sc0 : p == 1 ? sc1 : sc2);
                    // refill copies: 8-15 in an even block's first half, 0-7 in an
                    // odd block's second half, one per 16 MFMAs
                    const bool cp = H == 1 ? P == 1 : (P == 0 && !FIRST);
                    if constexpr (FN != 8) {
                        // Six fragment columns (six MFMA slots a row): the six B
                        // copies go out in the first six even rows; the next
                        // row's A plane takes slots 0-3 (done two MFMAs before
                        // that row); B plane p+1 of the six fragments spreads
                        // over the plane's slots 2-45; the next block's A
                        // fragment i is read at the last slot of row (3, i).
                        const int cq = (H == 1 ? 0 : 8) + (r % (2 * FM)) / 2;
                        if (cp && j == 0 && r % 2 == 0 && cq < FM + FN) copy_r4(cq);
                        if (p == 3) {
                            if (i == 0) fb[j] = *(const i32x4 *)(f + BOFF + (wn * FN + j) * 2048);
                            if (j == FN - 1) fa[i] = *(const i32x4 *)(f + (wm * FM + i) * 2048);
                        }
#pragma unroll
                        for (int k = 0; k < 6; ++k)
                            if (k < nops(pn) && k * 4 / nops(pn) == j) plane_op(pn, k, fa[in], ap[(r + 1) % 2]);
                        if (p < 3) {
                            const int g = i * FN + j, nk = nops(p + 1), nb = FN * nk;
#pragma unroll
                            for (int u = 0; u < FN * 6; ++u)
                                if (u < nb && 2 + u * 43 / nb == g)
                                    plane_op(p + 1, u % nk, fb[u / nk], bp[(p + 1) % 2][u / nk]);
                        } else if (i >= 1 && i - 1 < FN) {
                            if (j >= 2 && j < 6) plane_op(0, j - 2, fb[i - 1], bp[0][i - 1]);
                        }
                    } else {
                        if (cp && j == 0 && r % 2 == 0) copy_r4((H == 1 ? 0 : 8) + (r % (2 * FM)) / 2);
                        if (p == 3) {
                            // plane 3: the next block's fragments
                            if (i == 0) fb[j] = *(const i32x4 *)(f + BOFF + (wn * FN + j) * 2048);
                            if (j == 6) fa[i] = *(const i32x4 *)(f + (wm * FM + i) * 2048);
                        }
                        // A plane of the next row: slots 1 ..
                        if (j >= 1 && j - 1 < nops(pn)) plane_op(pn, j - 1, fa[in], ap[(r + 1) % 2]);
                        // B plane p+1 of fragment i (plane 3: the next block's plane 0
                        // of fragment i-1, and of fragment 7 too in row (3, 7))
                        if (p < 3) {
                            if (j >= 2 && j - 2 < nops(p + 1)) plane_op(p + 1, j - 2, fb[i], bp[(p + 1) % 2][i]);
                        } else if (i >= 1) {
                            if (j >= 2 && j < 6) plane_op(0, j - 2, fb[i - 1], bp[0][i - 1]);
                            if (i == FM - 1 && j >= 4) plane_op(0, j - 4, fb[FM - 1], bp[0][FM - 1]);
                        }
                    }
                }
            }
        };
        auto body1 = [&](auto par_c, auto first_c, int t) {
            half1(par_c, first_c, std::integral_constant<int, 0>{}, t);
            half1(par_c, first_c, std::integral_constant<int, 1>{}, t);
        };
        body1(P0{}, std::true_type{}, 0);
        int t = 1;
        for (; t + 1 < nk; t += 2) {
            body1(P1{}, F0{}, t);
            body1(P0{}, F0{}, t + 1);
        }
        if (t < nk) body1(P1{}, F0{}, t);
    }

    // The accumulators are read 32 wait states after the last MFMA.
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) asm volatile("" : "+a"(acc[i][j]));

    // Epilogue: lane holds C[m][n..n+3] of each fragment.  (Kept row by row:
    // hoisted across rows, the reads of the accumulators that need vector
    // work first, the int4 shift, crowd the vector registers.)
    const bool vec_ok = ((N | ldo) & 3) == 0;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        const int64_t m = m0 + wm * (16 * FM) + i * 16 + (lane % 16);
        if (m >= M) continue;
        const float *lds_sx = (const float *)(smem + 2 * SS);
        const float *lds_sw = lds_sx + BM;
        float scale_m = 0.f;
        if constexpr (KIND == KIND_LINEAR) scale_m = lds_sx[m - m0];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int64_t n = n0 + wn * (16 * FN) + j * 16 + (lane / 16) * 4;
            if (n >= N) continue;
            i32x4 v;
            if constexpr (KIND == KIND_B1F4) {
                // exact: the fp32 sums are integers below 2^24
                const f32x4 fv = __builtin_bit_cast(f32x4, acc[i][j]);
                v = i32x4{(int32_t)fv.x, (int32_t)fv.y, (int32_t)fv.z, (int32_t)fv.w};
            } else
                v = acc[i][j];
            if constexpr (KIND == KIND_S4) v = v >> 8;
            if constexpr (KIND == KIND_LINEAR) {
                float *o = (float *)out + m * (int64_t)ldo + n;
                if (vec_ok) {
                    const f32x4 s = *(const f32x4 *)(lds_sw + (n - n0));
                    f32x4 r;
                    r.x = ((float)v.x * scale_m) * s.x;
                    r.y = ((float)v.y * scale_m) * s.y;
                    r.z = ((float)v.z * scale_m) * s.z;
                    r.w = ((float)v.w * scale_m) * s.w;
                    *(f32x4 *)o = r;
                } else {
                    for (int r = 0; r < 4 && n + r < N; ++r) o[r] = ((float)v[r] * scale_m) * lds_sw[n - n0 + r];
                }
            } else {
                int32_t *o = (int32_t *)out + m * (int64_t)ldo + n;
                if (accumulate) {
                    for (int r = 0; r < 4 && n + r < N; ++r) atomicAdd(o + r, v[r]);
                } else if (vec_ok) {
                    *(i32x4 *)o = v;
                } else {
                    for (int r = 0; r < 4 && n + r < N; ++r) o[r] = v[r];
                }
            }
        }
    }
}

template <int KIND, int FM, int FN>
static hipError_t launch_w4(const void *A, const void *B, void *out, const float *sx, const float *sw,
                            int64_t M, int64_t N, int64_t Kb, int64_t ldo, int64_t ksplit, hipStream_t s)
{
    constexpr int64_t BM = 32 * FM, BN = 32 * FN;
    const uint64_t tm = (uint64_t)((M + BM - 1) / BM), tn = (uint64_t)((N + BN - 1) / BN);
    if (tm * tn > 0x7FFFFFFFull) return hipErrorInvalidValue;
    if (ksplit <= 0 || ksplit > Kb) ksplit = Kb;
    if (ksplit < Kb && (KIND == KIND_LINEAR || ksplit % 128 != 0)) return hipErrorInvalidValue;
    const uint32_t nsplit = (uint32_t)((Kb + ksplit - 1) / ksplit);
    hipLaunchKernelGGL((mfma_w4_kernel<KIND, FM, FN>), dim3((uint32_t)(tm * tn), nsplit), dim3(256), 0, s,
                       (const int8_t *)A, (const int8_t *)B, out, sx, sw, (int32_t)M, (int32_t)N,
                       (int32_t)Kb, (uint32_t)tm, (uint32_t)tn, (int32_t)ldo, (int32_t)ksplit);
    return hipGetLastError();
}

// ---- variant table --------------------------------------------------------
// index = 3*tile + (stages - 2); tile 0 = small, 1 = medium, 2 = large.
// Each tile has an LDS budget; the K depth of a stage (BK bytes) is chosen so
// that the stage count fits it: more stages hide more latency but take more
// LDS per workgroup and so allow fewer workgroups per CU, the trade-off of
// Research results item 1.  Measured on MI355X at 4096^3 int8: a medium tile
// with two 32 KiB stages (two workgroups per CU) runs in 66 us while the same
// tile with three 32 KiB stages (one workgroup per CU) needs 105 us, hence
// 64-byte stages for the deeper medium and large pipelines.
using S2 = MfmaCfg<64, 64, 128, 2, 2, 2>;     // 32 KiB
using S3 = MfmaCfg<64, 64, 128, 2, 2, 3>;     // 48 KiB
using S4 = MfmaCfg<64, 64, 128, 2, 2, 4>;     // 64 KiB
using SK64 = MfmaCfg<64, 64, 64, 2, 2, 2>;    // 16 KiB, convolutions with a short K
// The 2-stage medium tile runs 8 waves of 32x64 (two workgroups per CU): 3-16%
// faster than 4 waves of 64x64 on most shapes that choose it (4% slower at
// 1024 x 1024 x 4096); the 3- and 4-stage medium tiles lose with 8 waves and
// keep 4, as does the int4 convolution (its window gather, spread over twice
// the waves, made the 3x3 layer over 14x14x256 6% slower).
using M2 = MfmaCfg<128, 128, 128, 4, 2, 2>;   // 64 KiB
using M2W4 = MfmaCfg<128, 128, 128, 2, 2, 2>; // 64 KiB
using M3 = MfmaCfg<128, 128, 64, 2, 2, 3>;    // 48 KiB
using M4 = MfmaCfg<128, 128, 64, 2, 2, 4>;    // 64 KiB
// Large tile: 16 waves of 64x64 (L2W16, L4W16) or 8 waves of 64x128 (W8).
// Fewer, wider waves need fewer fragment reads and in-register conversions per
// MFMA (12 fragments per 32 MFMAs instead of 8 per 16) but hide less latency.
// Measured per variant, two builds timed in one process: the 3-stage large
// tile is 1-7% faster with 8 waves for every type, the 4-stage one 2-4% for
// int4 and mixed for int8, and the 2-stage one mixed for int8 and int4 (the
// 16 waves win by 4-9% when there are only 16-64 tiles).  The 1-bit tiles here
// use 8 waves throughout: their per-fragment bit work makes the wider wave
// tile pay at every depth (124 against 137 us at 4096 x 4096 x 8192 bits with
// the first bit expansion).  The 2-stage large tile of the int8, int4 and
// 1-bit (FP4 route) GEMMs and of the linear layer runs on the four-wave kernel
// (mfma_w4_kernel); the 1-bit int8 route and the convolutions keep the
// kernels above.
using L2W16 = MfmaCfg<256, 256, 128, 4, 4, 2>; // 128 KiB
using L2W8 = MfmaCfg<256, 256, 128, 4, 2, 2>;  // 128 KiB
using L3W8 = MfmaCfg<256, 256, 64, 4, 2, 3>;   // 96 KiB
using L4W16 = MfmaCfg<256, 256, 64, 4, 4, 4>;  // 128 KiB
using L4W8 = MfmaCfg<256, 256, 64, 4, 2, 4>;   // 128 KiB

template <class C, int KIND, bool CONV>
static hipError_t launch_one(const void *A, const void *B, void *out, const float *sx,
                             const float *sw, int64_t M, int64_t N, int64_t Kb, int64_t ldo,
                             int64_t ksplit, const ConvGeom &g, hipStream_t s)
{
    const uint64_t tm = (uint64_t)((M + C::BM - 1) / C::BM);
    const uint64_t tn = (uint64_t)((N + C::BN - 1) / C::BN);
    if (tm * tn > 0x7FFFFFFFull) return hipErrorInvalidValue;
    if (ksplit <= 0 || ksplit > Kb) ksplit = Kb;
    if (ksplit < Kb && (CONV || KIND == KIND_LINEAR || ksplit % C::BK != 0)) return hipErrorInvalidValue;
    const uint32_t nsplit = (uint32_t)((Kb + ksplit - 1) / ksplit);
    hipLaunchKernelGGL((mfma_gemm_kernel<C, KIND, CONV>), dim3((uint32_t)(tm * tn), nsplit), dim3(C::NT),
                       0, s, (const int8_t *)A, (const int8_t *)B, out, sx, sw, (int32_t)M, (int32_t)N,
                       (int32_t)Kb, (uint32_t)tm, (uint32_t)tn, (int32_t)ldo, (int32_t)ksplit, g);
    return hipGetLastError();
}

template <class C>
static void info_one(int *bm, int *bn, int *bk, int *st)
{
    *bm = C::BM; *bn = C::BN; *bk = C::BK; *st = C::ST;
}

template <int KIND, bool CONV>
static hipError_t dispatch(int variant, const void *A, const void *B, void *out, const float *sx,
                           const float *sw, int64_t M, int64_t N, int64_t Kb, int64_t ldo,
                           int64_t ksplit, const ConvGeom &g, hipStream_t s)
{
    switch (variant) {
    case 0: return launch_one<S2, KIND, CONV>(A, B, out, sx, sw, M, N, Kb, ldo, ksplit, g, s);
    case 1: return launch_one<S3, KIND, CONV>(A, B, out, sx, sw, M, N, Kb, ldo, ksplit, g, s);
    case 2: return launch_one<S4, KIND, CONV>(A, B, out, sx, sw, M, N, Kb, ldo, ksplit, g, s);
    case 3:
        return launch_one<std::conditional_t<CONV && KIND == KIND_S4, M2W4, M2>, KIND, CONV>(
            A, B, out, sx, sw, M, N, Kb, ldo, ksplit, g, s);
    case 4: return launch_one<M3, KIND, CONV>(A, B, out, sx, sw, M, N, Kb, ldo, ksplit, g, s);
    case 5: return launch_one<M4, KIND, CONV>(A, B, out, sx, sw, M, N, Kb, ldo, ksplit, g, s);
    default: break;
    }
    constexpr bool b1 = KIND == KIND_B1 || KIND == KIND_B1F4;
    switch (variant) {
    case 6:
        // int8, int4 and 1-bit (FP4 route) GEMMs and the linear layer: the
        // four-wave large tile (same 256x256 tile, two stages of 128 K-bytes).
        // 1-bit on the int8 route: 8 waves of 64x128; the convolutions: 16
        // waves of 64x64; the int4 GEMM under the A/B switch that keeps the
        // four-wave kernel to int8: 8 waves of 64x128.
        if constexpr ((KIND == KIND_S8 || KIND == KIND_LINEAR ||
                       ((KIND == KIND_S4 || KIND == KIND_B1F4) && !LB_AB_W4_INT8_ONLY)) && !CONV)
            return launch_w4<KIND, 8, 8>(A, B, out, sx, sw, M, N, Kb, ldo, ksplit, s);
        else
            return launch_one<std::conditional_t<b1 || (KIND == KIND_S4 && !CONV), L2W8, L2W16>, KIND, CONV>(
                A, B, out, sx, sw, M, N, Kb, ldo, ksplit, g, s);
    case 7: return launch_one<L3W8, KIND, CONV>(A, B, out, sx, sw, M, N, Kb, ldo, ksplit, g, s);
    case CONV_64x64_K64:
        // internal: the convolutions' small tile with 64-byte stages
        if constexpr (CONV) return launch_one<SK64, KIND, CONV>(A, B, out, sx, sw, M, N, Kb, ldo, ksplit, g, s);
        return hipErrorInvalidValue;
    case W4_256x192:
    case W4_192x256:
        // internal: the narrower four-wave tiles, int8 GEMM and linear layer
        // (both), int4 and 1-bit FP4-route GEMMs (256x192; under the A/B switch
        // that keeps the four-wave kernel to int8 they take variant 6's
        // 8-wave tile)
        if constexpr ((KIND == KIND_S8 || KIND == KIND_LINEAR) && !CONV) {
            if (variant == W4_256x192) return launch_w4<KIND, 8, 6>(A, B, out, sx, sw, M, N, Kb, ldo, ksplit, s);
            return launch_w4<KIND, 6, 8>(A, B, out, sx, sw, M, N, Kb, ldo, ksplit, s);
        } else if constexpr ((KIND == KIND_S4 || KIND == KIND_B1F4) && !CONV) {
            if (variant != W4_256x192) return hipErrorInvalidValue;
            if constexpr (LB_AB_W4_INT8_ONLY)
                return launch_one<L2W8, KIND, CONV>(A, B, out, sx, sw, M, N, Kb, ldo, ksplit, g, s);
            else
                return launch_w4<KIND, 8, 6>(A, B, out, sx, sw, M, N, Kb, ldo, ksplit, s);
        }
        return hipErrorInvalidValue;
    case 8:
        return launch_one<std::conditional_t<b1 || KIND == KIND_S4, L4W8, L4W16>, KIND, CONV>(
            A, B, out, sx, sw, M, N, Kb, ldo, ksplit, g, s);
    default: return hipErrorInvalidValue;
    }
}

// Zero n int32 values (the output of a split-K product, before its partial
// sums are added).  A kernel rather than hipMemsetAsync, so that a captured
// graph holds only kernel nodes.
__global__ __launch_bounds__(256) void zero_i32_kernel(int32_t *__restrict__ p, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) p[i] = 0;
}

hipError_t launch_zero_i32(int32_t *p, int64_t n, hipStream_t s)
{
    if (n <= 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, 8192);
    hipLaunchKernelGGL(zero_i32_kernel, dim3((uint32_t)blocks), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

hipError_t launch_mfma(int kind, int variant, const void *A, const void *B, void *out,
                       const float *sx, const float *sw, int64_t M, int64_t N, int64_t Kb,
                       int64_t ldo, int64_t ksplit, hipStream_t s)
{
    const ConvGeom none{};
    switch (kind) {
    case KIND_S8: return dispatch<KIND_S8, false>(variant, A, B, out, sx, sw, M, N, Kb, ldo, ksplit, none, s);
    case KIND_S4: return dispatch<KIND_S4, false>(variant, A, B, out, sx, sw, M, N, Kb, ldo, ksplit, none, s);
    case KIND_LINEAR:
        return dispatch<KIND_LINEAR, false>(variant, A, B, out, sx, sw, M, N, Kb, ldo, ksplit, none, s);
    case KIND_B1: return dispatch<KIND_B1, false>(variant, A, B, out, sx, sw, M, N, Kb, ldo, ksplit, none, s);
    case KIND_B1F4: return dispatch<KIND_B1F4, false>(variant, A, B, out, sx, sw, M, N, Kb, ldo, ksplit, none, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_conv(int kind, int variant, const void *X, const void *F, int32_t *Y,
                       int64_t M, int64_t N, int64_t Kb, const ConvGeom &g, hipStream_t s)
{
    switch (kind) {
    case KIND_S8: return dispatch<KIND_S8, true>(variant, X, F, Y, nullptr, nullptr, M, N, Kb, N, Kb, g, s);
    case KIND_S4: return dispatch<KIND_S4, true>(variant, X, F, Y, nullptr, nullptr, M, N, Kb, N, Kb, g, s);
    default: return hipErrorInvalidValue;
    }
}

int mfma_variant_info(int kind, int variant, int *bm, int *bn, int *bk_bytes, int *stages)
{
    (void)kind;  // the large tiles' wave count varies by type, not their shape
    switch (variant) {
    case 0: info_one<S2>(bm, bn, bk_bytes, stages); return 0;
    case 1: info_one<S3>(bm, bn, bk_bytes, stages); return 0;
    case 2: info_one<S4>(bm, bn, bk_bytes, stages); return 0;
    case 3: info_one<M2>(bm, bn, bk_bytes, stages); return 0;
    case 4: info_one<M3>(bm, bn, bk_bytes, stages); return 0;
    case 5: info_one<M4>(bm, bn, bk_bytes, stages); return 0;
    case 6: info_one<L2W16>(bm, bn, bk_bytes, stages); return 0;
    case 7: info_one<L3W8>(bm, bn, bk_bytes, stages); return 0;
    case 8: info_one<L4W16>(bm, bn, bk_bytes, stages); return 0;
    case W4_256x192: *bm = 256; *bn = 192; *bk_bytes = 128; *stages = 2; return 0;
    case CONV_64x64_K64: info_one<SK64>(bm, bn, bk_bytes, stages); return 0;
    case W4_192x256: *bm = 192; *bn = 256; *bk_bytes = 128; *stages = 2; return 0;
    default: return -1;
    }
}

}  // namespace lb
