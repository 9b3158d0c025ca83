// lb_device.hpp -- device-side building blocks shared by the gfx950 kernels:
// buffer resources, direct global->LDS copies, pipeline waits and the
// XCD-aware workgroup -> output-tile map.
//
// The kernels follow the thread-block-tiled GEMM described in the digest of
// "Leveraging Large-Scale Data for Efficient Low-Bit CUTLASS GEMM Optimization
// via Neural Networks" (Research results, item 1): C is cut into equal
// workgroup tiles, each tile loops over K reading matching slices of A and B,
// and a multi-stage pipeline overlaps the loads of later K slices with the math
// on the current one.  On gfx950 a pipeline stage is an LDS buffer filled by
// buffer_load ... lds (the copy engine writes LDS directly, no register
// staging), so S stages keep S-1 K slices in flight.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lb {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Raw buffer resource for gfx950: 48-bit base, stride 0, num_records bytes.
// Loads at offsets >= num_records return zero and touch no memory, so rows
// past the end of an operand are never read.
__device__ inline i32x4 make_rsrc(const void *base, uint64_t num_records)
{
    uint64_t b = (uint64_t)(uintptr_t)base;
    uint32_t n = num_records > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)num_records;
    i32x4 r;
    r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    r.y = __builtin_amdgcn_readfirstlane((int)((uint32_t)(b >> 32) & 0xFFFFu));
    r.z = __builtin_amdgcn_readfirstlane((int)n);
    r.w = 0x00020000;
    return r;
}

// One wave-wide 16-byte-per-lane copy from global memory straight into LDS:
// lane i's 16 bytes at rsrc.base + voff land at LDS byte lds_base + 16*i.  The
// compiler does not see this LDS write (it would otherwise wait for every
// outstanding copy before any LDS read, collapsing the pipeline); the kernels
// order it explicitly with wait_vm_barrier().  On gfx9-family parts an LDS
// copy must not read M0 in the instruction right after the SALU write that set
// it, hence the s_nop between the two.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ inline void dma16(i32x4 rsrc, uint32_t voff, uint32_t lds_base)
{
    asm volatile("s_mov_b32 m0, %2\n\t"
                 "s_nop 0\n\t"
                 "buffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(lds_base)
                 : "memory", "m0");
}
// The same with 4 bytes per lane: lane i's word lands at LDS byte lds_base + 4*i.
__device__ inline void dma4(i32x4 rsrc, uint32_t voff, uint32_t lds_base)
{
    asm volatile("s_mov_b32 m0, %2\n\t"
                 "s_nop 0\n\t"
                 "buffer_load_dword %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(lds_base)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// The same 16 bytes per lane loaded into registers, from a resource made by
// make_rsrc (for A/B builds that stage operands through registers); offsets
// >= num_records read zero.
__device__ inline i32x4 load16(i32x4 rsrc, uint32_t voff)
{
    const uint64_t b = (uint64_t)(uint32_t)rsrc.x | ((uint64_t)((uint32_t)rsrc.y & 0xFFFFu) << 32);
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc((void *)(uintptr_t)b, (short)0, rsrc.z, rsrc.w);
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0);
}

// Wait until at most N of this wave's copies are outstanding and its LDS reads
// have returned, then barrier: afterwards every wave's copies older than the
// last N (per wave) are visible in LDS, and no wave still reads the buffer the
// next copy will overwrite.
template <int N>
__device__ inline void wait_vm_barrier()
{
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "n"(N) : "memory");
}

__device__ inline void wait_vm_all()
{
    asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
}

__device__ inline void barrier_lds()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
}

// LDS address (byte offset in the workgroup's LDS) of a __shared__ object.
__device__ inline uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)p;
}

// Workgroup -> output tile.  Consecutive workgroup ids are dispatched round
// robin over the 8 XCDs of an MI355X, each with its own L2.  First give each
// XCD a contiguous run of tile ids, then walk tiles in bands of `group` tile
// rows so that the tiles an XCD holds at one time share rows of A and columns
// of B in its L2.  The band height also sets which rows of A and columns of B
// all XCDs read at the same time through the shared last-level cache; it was
// chosen per tile size from measurements (4 for the medium and large tiles, 8
// for the small one).
// (LB_AB_TILE_MAP_PLAIN=1, set only by A/B profiling builds: plain row-major
// tile order instead.)
#ifndef LB_AB_TILE_MAP_PLAIN
#define LB_AB_TILE_MAP_PLAIN 0
#endif
__device__ inline void tile_of_block(uint32_t bid, uint32_t tiles_m, uint32_t tiles_n,
                                     uint32_t group, uint32_t &tm, uint32_t &tn)
{
    if (LB_AB_TILE_MAP_PLAIN) {
        tm = bid / tiles_n;
        tn = bid % tiles_n;
        return;
    }
    const uint32_t T = tiles_m * tiles_n;
    const uint32_t q = T / 8u, r = T % 8u;
    const uint32_t xcd = bid % 8u, idx = bid / 8u;
    const uint32_t id = (xcd < r) ? xcd * (q + 1u) + idx : r * (q + 1u) + (xcd - r) * q + idx;
    const uint32_t per_band = group * tiles_n;
    const uint32_t band = id / per_band;
    const uint32_t first = band * group;
    const uint32_t rows = min(group, tiles_m - first);
    const uint32_t in_band = id - band * per_band;
    tm = first + in_band % rows;
    tn = in_band / rows;
}

}  // namespace lb
