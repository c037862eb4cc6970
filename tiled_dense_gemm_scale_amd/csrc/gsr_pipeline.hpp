// gsr_pipeline.hpp -- the pieces every kernel here that copies operands
// global -> LDS by the buffer unit itself (no register staging) shares: the
// raw buffer descriptor, the direct-to-LDS copy, the waits on the copies, the
// LDS barrier and the LDS chunk swizzles.
//
// Design notes (CDNA4 / gfx950):
//  * buffer_load_dwordx4 ... lds writes lane L's 16 bytes to LDS at
//    base + 16*L.  Every wave-wide copy therefore fills 1 KiB of LDS
//    contiguously; the bank-conflict swizzle is applied on the global side by
//    choosing which 16-byte chunk each lane fetches.  Out-of-range chunks
//    (ragged M, N or K) read as zero, so the tile maths never sees garbage.
//  * A is K-contiguous and lands as [BM][BK] rows; a lane's MFMA operand is
//    one 128-bit LDS read.
//  * B is N-contiguous and lands as [BK][BN] rows.  ds_read_b64_tr_b16 gives,
//    within each 16-lane group, output lane i element e = source lane
//    (4e + i/4) element (i % 4): when source lane 4e+q points at row k0+e,
//    columns n0+4q..n0+4q+3, lane i receives B[k0..k0+3][n0+i], i.e. four
//    K-consecutive values of one column.  Two such reads form the eight
//    values of an MFMA operand.
//  * The MFMA takes B^T as its first operand and A^T as its second, so an
//    accumulator block holds four consecutive n per lane and register group.
#pragma once

#include "gsr_kernels.hpp"

namespace gsr {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

typedef int i32x4 __attribute__((ext_vector_type(4)));

// The copies, the waits on them and the barrier are issued as inline asm with
// a "memory" clobber: the compiler then neither hoists LDS reads across them
// nor adds its own conservative vmcnt(0) waits (it would otherwise wait for
// every outstanding copy before each LDS read, which serialises the ring).
// Vector-memory operations retire in order, so waits the compiler emits for
// its own loads can only become stricter, never wrong.

// Buffer resource for a raw byte range (gfx9-family descriptor: base address,
// stride 0, num_records = bytes, data-format word).
__device__ __forceinline__ i32x4 raw_rsrc(const void* p, uint32_t bytes)
{
    const uint64_t a = (uint64_t)(uintptr_t)p;
    i32x4 r;
    r[0] = (int)(uint32_t)a;
    r[1] = (int)((uint32_t)(a >> 32) & 0xffffu);
    r[2] = (int)bytes;
    r[3] = 0x00020000;
    return r;
}

// Copy 16 bytes per lane from the buffer at byte offset voff (out of range
// reads zero) into LDS at lds_addr + 16 * lane.
__device__ __forceinline__ void copy16_to_lds(i32x4 rsrc, uint32_t voff, uint32_t lds_addr)
{
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :: "v"(voff), "s"(rsrc), "s"(lds_addr) : "memory", "m0");
}

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

__device__ __forceinline__ void wait_vmcnt_dyn(int n)
{
    // n is uniform and small; fall back to stricter waits past 8
    if (n <= 0) wait_vmcnt<0>();
    else if (n == 1) wait_vmcnt<1>();
    else if (n == 2) wait_vmcnt<2>();
    else if (n == 3) wait_vmcnt<3>();
    else if (n < 6) wait_vmcnt<4>();
    else if (n < 8) wait_vmcnt<6>();
    else if (n < 12) wait_vmcnt<8>();
    else if (n < 16) wait_vmcnt<12>();
    else if (n < 24) wait_vmcnt<16>();
    else if (n < 32) wait_vmcnt<24>();
    else wait_vmcnt<32>();
}

// Barrier after this wave's LDS reads have returned (so no wave refills a
// buffer another wave is still reading).
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ uint32_t lds_address(const void* p)
{
    return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const uint8_t*)p);
}

// A tile rows of BK halves: 16-byte chunk c of row r sits at chunk c ^ swz_a(r).
template <int CH>
__device__ __forceinline__ uint32_t swz_a(uint32_t r)
{
    if constexpr (CH == 8) return (r ^ (r >> 3)) & 7u;
    else return ((r >> 1) ^ (r >> 2)) & 3u;  // CH == 4
}

// B tile rows (one k each) of BN halves: chunk c of row k sits at c ^ swz_b(k).
// A transpose read hands each 16-lane group rows k..k+3 of a 16-k substep
// (k = 8g' + 4r, g' = lane group / 2) and two 16-byte chunks per row, the
// group next to it the next two chunks of the same rows.
//  * 128-byte rows (BN = 64): the LDS serves 64 banks of 4 bytes per cycle,
//    so even rows fall on one half of the banks and odd rows on the other, and
//    rows k and k + 8 are read by the same instruction.  Masks (2(k mod 4)) ^
//    (2 if k mod 16 >= 8) give the rows served together disjoint chunks
//    whether the cycle takes lanes 0-31 (rows k..k+3, four chunks each) or
//    lanes 0-15 with 32-47 (rows k..k+3 and k+8..k+11, two chunks each), and
//    also when 16 lanes are served per cycle.  The masks 0, 6, 2, 4 by
//    k mod 4 used before repeat every four rows, which left rows k and k + 2
//    (and k and k + 8) on the same banks: two extra cycles per read
//    (rocprofv3 SQ_LDS_BANK_CONFLICT, one cycle per LDS instruction on the
//    64x64 K-split kernel at 1024^3).
//  * other widths: four consecutive rows get XOR masks whose bits 1-2 and
//    bits 2-3 are both distinct, which spreads a read's 4 rows x 2-4 chunks
//    over the banks.
template <int CHN>
__device__ __forceinline__ uint32_t swz_b(uint32_t k)
{
    if constexpr (CHN == 8) return ((k & 3u) << 1) ^ ((k >> 2) & 2u);
    const uint32_t e = k & 3u;
    const uint32_t f = ((e & 1u) * 6u) ^ ((e >> 1) * 10u);  // 0, 6, 10, 12
    return f & (uint32_t)(CHN - 1);
}

}  // namespace gsr
