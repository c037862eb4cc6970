// gsr_interleave.hpp -- the explicit-interleave design of the large-tile
// 128-bit kernels and the pieces they share.
//
// A workgroup owns one output tile with four MFMA waves, whose accumulators
// sit in AGPRs.  In the 256x256 kernels the register file gives one wave per
// SIMD, so nothing else hides a gap in the MFMA stream: every other
// instruction of a K-step is placed
// between MFMAs, one schedule unit (an MFMA plus its companions) at a time,
// with a scheduling barrier between units so the compiler keeps that order.
// Operand reads are 128-bit (A and B^T both K-contiguous in LDS, 16-byte
// chunks XOR-swizzled by row); A is copied straight into LDS by the buffer
// unit (buffer_load ... lds); B, stored N-contiguous, is loaded into
// registers one block per thread, transposed with byte permutes and written
// K-contiguous, or in the kernels of gsr_interleave16d.hpp and
// gsr_interleave16c.hpp copied into LDS as stored and read with transpose
// reads (the latter with four more waves that only issue the copies).  Both
// operands are requested two K-steps ahead (three in the 128x128 tile, which
// keeps a ring of four stages) through buffer descriptors that advance along
// K in SGPRs, so the compiler adds no waits of its own; the vmcnt
// bookkeeping is explicit.
// One barrier per K-step publishes the next step's buffers and frees the
// current ones.  The kernels on this design: 256x256, 128x256 and 128x128
// tiles on 16x16x32 MFMAs (gsr_interleave16.hpp, gsr_interleave16d.hpp,
// gsr_interleave16c.hpp).
//
// Ragged edges: rows of A past M and rows of B past K fall outside the
// advancing descriptors (read as zero); B columns past N and A columns past K
// get an out-of-range offset per lane; stores outside C are dropped.  K is
// walked in an even number of steps (the 128x128 ring: one by one): a step
// wholly past K multiplies zeros.
#pragma once

#include <type_traits>

#include "gsr_pipeline.hpp"

namespace gsr {

// The 256x256 tile of the design: four waves of 128x128, two LDS stages of A
// and B (the 16x16x32 kernels derive their configurations from it).
struct IlvCfg {
    static constexpr int BM = 256, BN = 256, BK = 64, WM = 2, WN = 2;
    static constexpr int NW = WM * WN, NT = kWave * NW;
    static constexpr int CH = BK / 8;
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
    static constexpr int B_REGION = 2 * A_BYTES;
    static constexpr int LDS_BYTES = 2 * (A_BYTES + B_BYTES);
    static constexpr int A_PER = A_BYTES / 1024 / NW;  // 8 copies per wave per step
    static constexpr int B_LOADS = 8;                  // one 8x8 block per thread
    static_assert((BK / 8) * (BN / 8) == NT, "one B block per thread");
    static_assert(A_PER == 8, "the unit plan places 8 copies");
};

// 16-byte global load into registers through a buffer descriptor (no compiler
// wait is attached: see wait_vmcnt_b).
__device__ __forceinline__ u32x4 load16(i32x4 rsrc, uint32_t voff)
{
    u32x4 v;
    asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen" : "=v"(v) : "v"(voff), "s"(rsrc) : "memory");
    return v;
}

// Wait for the vector-memory counter and tie the B registers to the wait, so
// no use of them is scheduled before their data is in.
template <int N>
__device__ __forceinline__ void wait_vmcnt_b(u32x4 (&r)[8])
{
    asm volatile("s_waitcnt vmcnt(%8)"
                 : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]), "+v"(r[4]), "+v"(r[5]), "+v"(r[6]), "+v"(r[7])
                 : "n"(N)
                 : "memory");
}

__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

}  // namespace gsr
