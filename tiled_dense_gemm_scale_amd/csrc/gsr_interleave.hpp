// gsr_interleave.hpp -- the explicit-interleave design of the large-tile
// 128-bit kernels and the pieces they share.
//
// A workgroup owns one output tile with four waves, whose accumulators sit in
// AGPRs.  The LDS footprint gives one wave per SIMD, so nothing else hides a
// gap in the MFMA stream: every other instruction of a K-step is placed
// between MFMAs, one schedule unit (an MFMA plus its companions) at a time,
// with a scheduling barrier between units so the compiler keeps that order.
// Operand reads are 128-bit (A and B^T both K-contiguous in LDS, 16-byte
// chunks XOR-swizzled by row); A is copied straight into LDS by the buffer
// unit (buffer_load ... lds); B, stored N-contiguous, is loaded into
// registers one block per thread, transposed with byte permutes and written
// K-contiguous, or in the kernel of gsr_interleave16d.hpp copied into LDS as
// stored and read with transpose reads.  Both operands are requested two
// K-steps ahead through buffer descriptors that advance along K in SGPRs, so
// the compiler adds no waits of its own; the vmcnt bookkeeping is explicit.
// One barrier per K-step publishes the next step's buffers and frees the
// current ones.  The kernels on this design: 128x128 tiles on 32x32x16
// MFMAs (gsr_interleave_q.hpp), 256x256 and 128x256 tiles on 16x16x32 MFMAs
// (gsr_interleave16.hpp, gsr_interleave16d.hpp, gsr_interleave16c.hpp).
//
// Ragged edges: rows of A past M and rows of B past K fall outside the
// advancing descriptors (read as zero); B columns past N and A columns past K
// get an out-of-range offset per lane; stores outside C are dropped.  K is
// walked in an even number of steps: a step wholly past K multiplies zeros.
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
    static constexpr int TM = WTM / 32, TN = WTN / 32;  // 4 x 4 accumulator blocks
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

// The epilogue of the interleaved kernels: scale, ReLU (or the variant: scale,
// bias, activation) and round in registers, then pass each wave's WTM x WTN
// fp16 sub-tile through its own WTM x 2*WTN bytes of LDS so that the global
// stores write whole row segments (WTN/8 lanes of 16 bytes per row) instead of
// 16 bytes in each of 32 rows.  16-byte chunk c of row r sits at physical
// chunk c ^ (r % (WTN/8)).  Called once every wave's copies have been drained.
template <class T = IlvCfg>
__device__ __forceinline__ void ilv_epilogue(const Problem& p, const f32x16 (&acc)[T::TN][T::TM],
                                             uint8_t* smem, int m0, int n0, int wm, int wn, int wave,
                                             uint32_t frow, uint32_t fhi)
{
    constexpr int TM = T::TM, TN = T::TN;
    const uint32_t lane = (uint32_t)(threadIdx.x & 63);
    const uint32_t N = (uint32_t)p.N;
    static_assert(T::NW * T::WTM * T::WTN * 2 <= T::LDS_BYTES, "epilogue tile fits");
    constexpr uint32_t CPR = T::WTN / 8, RB = T::WTN * 2;  // chunks and bytes per staging row
    static_assert((T::WTN == 128 || T::WTN == 64) && T::WTM % 32 == 0, "staging rows of 8 or 16 chunks");
    // The variant's bias values for the lane's 16 column groups are requested
    // before the barrier, so their latency overlaps it.
    const bool plain = plain_epilogue(p);
    f32x4 bvs[TN][4];
    {
        const __amdgpu_buffer_rsrc_t rbias = bias_rsrc(p);
        const bool load = !plain && p.bias != nullptr;
#pragma unroll
        for (int a = 0; a < TN; ++a)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                bvs[a][g] = load ? bias4(rbias, n0 + wn * T::WTN + a * 32 + 8 * g + 4 * (int)fhi)
                                 : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    lds_barrier();  // every wave is past its last operand read
    const float alpha = p.alpha;
    uint8_t* const ep = smem + wave * (T::WTM * T::WTN * 2);
    auto stage4 = [&](int a, int b, int g, half4 h) {
        const uint32_t r = (uint32_t)b * 32u + frow;
        const uint32_t c = ((uint32_t)(4 * a + g)) ^ (r & (CPR - 1u));
        *(u32x2*)(ep + r * RB + c * 16u + fhi * 8u) = __builtin_bit_cast(u32x2, h);
    };
    if (plain) {
#pragma unroll
        for (int a = 0; a < TN; ++a) {
#pragma unroll
            for (int b = 0; b < TM; ++b) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    half4 h;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float v = acc[a][b][4 * g + i] * alpha;
                        h[i] = (_Float16)(v > 0.0f ? v : 0.0f);
                    }
                    stage4(a, b, g, h);
                }
            }
        }
    } else {
        // act(alpha * acc + bias)
        with_activation(p.act, [&](auto act_tag) {
            constexpr int ACT = decltype(act_tag)::value;
#pragma unroll
            for (int a = 0; a < TN; ++a) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const f32x4 bv = bvs[a][g];
#pragma unroll
                    for (int b = 0; b < TM; ++b) {
                        const f32x16 av = acc[a][b];
                        f32x4 sv;
#pragma unroll
                        for (int i = 0; i < 4; ++i) sv[i] = av[4 * g + i];
                        stage4(a, b, g, epilogue4<ACT>(sv, alpha, bv));
                    }
                }
            }
        });
    }
    // The reads below take what other lanes of this wave wrote: LDS keeps a
    // wave's accesses in order, so only the compiler must not move them.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.C, (uint32_t)p.M * N * 2u);
    constexpr uint32_t RPI = 64u / CPR;  // rows per store instruction
    const uint32_t sc = (uint32_t)lane & (CPR - 1u);
    const int n = n0 + wn * T::WTN + 8 * (int)sc;
#pragma unroll
    for (int j = 0; j < (int)(T::WTM / RPI); ++j) {
        const uint32_t r = RPI * (uint32_t)j + (uint32_t)lane / CPR;
        const u32x4 v = *(const u32x4*)(ep + r * RB + ((sc ^ (r & (CPR - 1u))) << 4));
        const int m = m0 + wm * T::WTM + (int)r;
        const uint32_t off = ((m < p.M) & (n < p.N)) ? ((uint32_t)m * N + (uint32_t)n) * 2u : kOutOfRange;
        __builtin_amdgcn_raw_buffer_store_b128(v, rc, off, 0, 0);
    }
}

}  // namespace gsr
