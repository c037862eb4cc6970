// gsr_interleave.hpp -- the large-tile 128-bit path of C = ReLU(alpha * A @ B)
// with an explicit instruction interleave.
//
// A 256x256 tile per workgroup, four waves each owning 128x128 of it (256 fp32
// accumulators per lane, held in AGPRs).  The LDS footprint (2 x 64 KiB) gives
// one wave per SIMD, so nothing else hides a gap in the MFMA stream: every
// other instruction of a K-step is placed between MFMAs, one schedule unit
// (an MFMA plus its companions) at a time, with a scheduling barrier between
// units so the compiler keeps that order.
//
// Per K-step t (BK = 64, four 16-k substeps of 16 MFMAs each), units carry:
//   substep 0: the next substep's operand reads, then the byte-permute
//              transpose of the B block of step t+1;
//   substep 1: the next substep's operand reads alternating with the B loads
//              of step t+2;
//   substep 2: the next substep's operand reads alternating with the
//              transposed B writes of step t+1;
//   substep 3: four MFMAs, the wait + barrier that publishes step t+1's
//              buffers, then the first operand reads of step t+1 and the A
//              copies of step t+2 (buffer_load ... lds) into the stage that
//              the barrier freed.
// Both operands are thus requested about three substeps before they are
// needed, which hides an L2 miss.
// Operand reads are all 128-bit (A and B both K-contiguous in LDS, 16-byte
// chunks XOR-swizzled by row), and global traffic is issued as inline asm on
// buffer descriptors that advance in SGPRs, so the compiler adds no waits of
// its own; the vmcnt bookkeeping is explicit below.
//
// Ragged edges: rows of A past M and rows of B past K fall outside the
// advancing descriptors (read as zero); B columns past N and A columns past K
// get an out-of-range offset per lane; stores outside C are dropped.  K is
// walked in an even number of steps: a step wholly past K multiplies zeros.
#pragma once

#include <type_traits>

#include "gsr_pipeline.hpp"

namespace gsr {

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

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_scale_relu_ilv_kernel(Problem p)
{
    using T = IlvCfg;
    constexpr int BK = T::BK, CH = T::CH, TM = T::TM, TN = T::TN;

    __shared__ __attribute__((aligned(1024))) uint8_t smem[T::LDS_BYTES];  // A0 | A1 | B0 | B1

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / T::WN, wn = wave % T::WN;

    int tm, tn;
    tile_of(blockIdx.x, gridDim.x, p, tm, tn);
    const int m0 = tm * T::BM, n0 = tn * T::BN;
    const uint32_t K = (uint32_t)p.K, N = (uint32_t)p.N;
    const uint32_t lds0 = lds_address(smem);

    // ---- descriptors that advance along K ---------------------------------
    // A: base at (m0, k0), records up to the end of A: rows >= M are out.
    uint64_t a_base = (uint64_t)(uintptr_t)p.A + ((uint64_t)m0 * K) * 2u;
    uint32_t a_recs = ((uint32_t)p.M * K - (uint32_t)m0 * K) * 2u;
    // B: base at (k0, n0), records up to the end of B: rows >= K are out.
    uint64_t b_base = (uint64_t)(uintptr_t)p.B + (uint64_t)n0 * 2u;
    uint32_t b_recs = (K * N - (uint32_t)n0) * 2u;
    auto rsrc_of = [](uint64_t base, uint32_t recs) {
        i32x4 r;
        r[0] = (int)(uint32_t)base;
        r[1] = (int)((uint32_t)(base >> 32) & 0xffffu);
        r[2] = (int)recs;
        r[3] = 0x00020000;
        return r;
    };
    // Descriptors positioned at column k of A / row k of B; from k = K on they
    // cover no bytes at all, so every access through them reads zero.
    auto a_rsrc = [&](uint32_t k) { return (k < K) ? rsrc_of(a_base + (uint64_t)k * 2u, a_recs - k * 2u) : rsrc_of(a_base, 0u); };
    auto b_rsrc = [&](uint32_t k) {
        return (k < K) ? rsrc_of(b_base + (uint64_t)k * N * 2u, b_recs - k * N * 2u) : rsrc_of(b_base, 0u);
    };

    // ---- per-lane copy plan ------------------------------------------------
    // A copy i of this wave fills LDS chunk positions 64*(wave+4i) + lane:
    // row P / 8, physical chunk P % 8, logical chunk c = physical ^ swz(row).
    uint32_t a_voff[T::A_PER], a_kc[T::A_PER];
#pragma unroll
    for (int i = 0; i < T::A_PER; ++i) {
        const uint32_t P = 64u * (uint32_t)(wave + i * T::NW) + (uint32_t)lane;
        const uint32_t r = P / CH;
        const uint32_t c = (P % CH) ^ swz_a<CH>(r);
        a_voff[i] = (r * K + 8u * c) * 2u;
        a_kc[i] = 8u * c;
    }
    // B block of this thread: rows kb*8..+7, columns nb*8..+7 of the tile.
    const uint32_t kb = (uint32_t)tid / (T::BN / 8), nb = (uint32_t)tid % (T::BN / 8);
    uint32_t b_voff[8];
    {
        const bool nok = (uint32_t)n0 + nb * 8u < N;
#pragma unroll
        for (int j = 0; j < 8; ++j) b_voff[j] = nok ? ((kb * 8u + (uint32_t)j) * N + nb * 8u) * 2u : kOutOfRange;
    }
    // transposed B writes: column nb*8+j of the tile, chunk kb
    uint32_t bw_addr[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t r = nb * 8u + (uint32_t)j;
        bw_addr[j] = (uint32_t)T::B_REGION + r * (BK * 2) + ((kb ^ swz_a<CH>(r)) << 4);
    }
    // operand reads: lane l reads row (l % 32) of a 32-row block, chunk
    // 2*ks + l/32 of the row (stage 0 addresses; stage 1 adds a constant)
    const uint32_t frow = lane & 31, fhi = lane >> 5;
    uint32_t x_addr[4][TN], y_addr[4][TM];
#pragma unroll
    for (int a = 0; a < TN; ++a) {
        const uint32_t r = wn * T::WTN + a * 32 + frow;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            x_addr[ks][a] = (uint32_t)T::B_REGION + r * (BK * 2) + (((2u * ks + fhi) ^ swz_a<CH>(r)) << 4);
    }
#pragma unroll
    for (int b = 0; b < TM; ++b) {
        const uint32_t r = wm * T::WTM + b * 32 + frow;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) y_addr[ks][b] = r * (BK * 2) + (((2u * ks + fhi) ^ swz_a<CH>(r)) << 4);
    }

    f32x16 acc[TN][TM];
#pragma unroll
    for (int a = 0; a < TN; ++a)
#pragma unroll
        for (int b = 0; b < TM; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

    half8 xf[2][TN], yf[2][TM];  // two operand sets: substep parity
    u32x4 breg[8];               // B block of a future step
    u32x4 bcol[8];               // its transpose

    // ---- building blocks ---------------------------------------------------
    // A copy i of step "k0" into stage S (k0 in elements; the descriptor is at k0).
    auto copy_a = [&](int S, int i, uint32_t kleft, const i32x4& ra) {
        const uint32_t off = (a_kc[i] < kleft) ? a_voff[i] : kOutOfRange;
        copy16_to_lds(ra, off, lds0 + (uint32_t)(S * T::A_BYTES) + (uint32_t)(wave + i * T::NW) * 1024u);
    };
    auto read_x = [&](int S, int ks, int a, half8& dst) {
        dst = __builtin_bit_cast(half8, *(const u32x4*)(smem + S * T::B_BYTES + x_addr[ks][a]));
    };
    auto read_y = [&](int S, int ks, int b, half8& dst) {
        dst = __builtin_bit_cast(half8, *(const u32x4*)(smem + S * T::A_BYTES + y_addr[ks][b]));
    };
    // read i (0..7) of the next substep's operands, in the order its MFMAs
    // need them: x0, y0..y3 (units 0-3 use x0 with every y), then x1..x3
    auto read_next = [&](int S, int ks, int i, half8 (&xs)[TN], half8 (&ys)[TM]) {
        if (i == 0) read_x(S, ks, 0, xs[0]);
        else if (i <= TM) read_y(S, ks, i - 1, ys[i - 1]);
        else read_x(S, ks, i - TM, xs[i - TM]);
    };
    auto mma = [&](int i, const half8 (&xs)[TN], const half8 (&ys)[TM]) {
        const int a = i / TM, b = i % TM;
        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(xs[a], ys[b], acc[a][b], 0, 0, 0);
    };

    // One K-step on stage S (the step's A and B are in LDS stage S, its
    // substep-0 operands are in xf[0]/yf[0]).  t is the step index.  Loads run
    // two steps ahead: B(t+2) is loaded in substep 1 (once the transpose has
    // freed breg) and A(t+2) is copied into stage S in substep 3 (once the
    // barrier has freed it), so each has about three substeps of MFMA work to
    // arrive in.
    auto step = [&](auto stage_tag, int t) {
        constexpr int S = decltype(stage_tag)::value;
        constexpr int SN = S ^ 1;
        const uint32_t k2 = (uint32_t)(t + 2) * BK;

        // substep 0: reads for substep 1 on even units; from unit 8 the
        // transpose of B(t+1), whose loads are in once at most the 8 copies of
        // A(t+1) issued after them are still in flight
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            mma(i, xf[0], yf[0]);
            if ((i & 1) == 0) read_next(S, 1, i >> 1, xf[1], yf[1]);
            if (i == 8) wait_vmcnt_b<T::A_PER>(breg);
            if (i >= 8) {
                // 4 of the 32 permutes per unit
                const int e = (i - 8) >> 1, d0 = ((i - 8) & 1) * 2;
#pragma unroll
                for (int d = d0; d < d0 + 2; ++d) {
                    bcol[2 * d][e] = pack_lo(breg[2 * e][d], breg[2 * e + 1][d]);
                    bcol[2 * d + 1][e] = pack_hi(breg[2 * e][d], breg[2 * e + 1][d]);
                }
            }
            sched_fence();
        }
        // substep 1: reads for substep 2 on even units, the loads of B(t+2)
        // on odd units
        {
            const i32x4 rb = b_rsrc(k2);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                mma(i, xf[1], yf[1]);
                if ((i & 1) == 0) read_next(S, 2, i >> 1, xf[0], yf[0]);
                else breg[i >> 1] = load16(rb, b_voff[i >> 1]);
                sched_fence();
            }
        }
        // substep 2: reads for substep 3 on even units, the transposed B(t+1)
        // stores into stage SN on odd units (the LDS work of a step then
        // spreads as 8 / 8 / 16 / 16 operations over its four substeps)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            mma(i, xf[0], yf[0]);
            if ((i & 1) == 0) read_next(S, 3, i >> 1, xf[1], yf[1]);
            else *(u32x4*)(smem + SN * T::B_BYTES + bw_addr[i >> 1]) = bcol[i >> 1];
            sched_fence();
        }
        // substep 3: publish step t+1 (the copies of A(t+1) landed: only the 8
        // B(t+2) loads issued after them may be in flight; B(t+1) stores are
        // done; every read of stage S finished), then the substep-0 reads of
        // step t+1 and the copies of A(t+2) into the freed stage S
        {
            const uint32_t kleft2 = (k2 < K) ? K - k2 : 0u;  // valid k in step t+2
            const i32x4 ra = a_rsrc(k2);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                mma(i, xf[1], yf[1]);
                if (i == 3) {
                    wait_vmcnt<T::B_LOADS>();
                    lds_barrier();
                }
                if (i >= 4 && i < 12) {
                    read_next(SN, 0, i - 4, xf[0], yf[0]);
                    copy_a(S, i - 4, kleft2, ra);
                }
                sched_fence();
            }
        }
    };

    // ---- prologue: A(0), B(0) in stage 0; B(1) and then A(1) in flight ------
    const int ksteps = (((int)K + BK - 1) / BK + 1) & ~1;  // even
    {
        const i32x4 ra0 = a_rsrc(0);
#pragma unroll
        for (int i = 0; i < T::A_PER; ++i) copy_a(0, i, K, ra0);
        const i32x4 rb = b_rsrc(0);
#pragma unroll
        for (int j = 0; j < 8; ++j) breg[j] = load16(rb, b_voff[j]);
        wait_vmcnt_b<0>(breg);
        transpose8x8(breg, bcol);
#pragma unroll
        for (int j = 0; j < 8; ++j) *(u32x4*)(smem + bw_addr[j]) = bcol[j];
        const i32x4 rb1 = b_rsrc((uint32_t)BK);
#pragma unroll
        for (int j = 0; j < 8; ++j) breg[j] = load16(rb1, b_voff[j]);
        const uint32_t kleft1 = ((uint32_t)BK < K) ? K - (uint32_t)BK : 0u;
        const i32x4 ra1 = a_rsrc((uint32_t)BK);
#pragma unroll
        for (int i = 0; i < T::A_PER; ++i) copy_a(1, i, kleft1, ra1);
        lds_barrier();
#pragma unroll
        for (int i = 0; i < 8; ++i) read_next(0, 0, i, xf[0], yf[0]);
    }

    for (int t = 0; t < ksteps; t += 2) {
        step(std::integral_constant<int, 0>{}, t);
        step(std::integral_constant<int, 1>{}, t + 1);
    }
    // Drain every load before the epilogue: no copy may land in LDS after the
    // workgroup is gone, and tying the B registers keeps the compiler from
    // reusing them while the last (dead) loads into them are in flight.
    wait_vmcnt_b<0>(breg);

    // ---- epilogue ------------------------------------------------------------
    ilv_epilogue(p, acc, smem, m0, n0, wm, wn, wave, frow, fhi);
}

}  // namespace gsr
