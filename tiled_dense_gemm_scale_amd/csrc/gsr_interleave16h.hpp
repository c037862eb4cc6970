// gsr_interleave16h.hpp -- the 128x256 explicitly interleaved kernel on the
// 16x16x32 fp16 MFMA with B transposed through registers: the twin of the
// 128x256 kernel in gsr_interleave16d.hpp (B copied to LDS), which gives the
// same bits faster; kept for comparison.
//
// Four waves of 64x128, A copied straight into LDS, B one 8x8 block per
// thread through registers, both operands two K-steps ahead, one barrier per
// K-step, with the matrix instruction, operand fragments, register sets and
// LDS chunk order of the 256x256 16x16x32 kernel in gsr_interleave16.hpp.
//
// Each wave owns 64x128 of the tile as 8 (n) x 4 (m) accumulator blocks of
// 16x16 (128 fp32 per lane, in AGPRs).  A K-step is two 32-deep substeps of
// 32 MFMAs; MFMA slot i of a substep multiplies B^T fragment X[i / 4] with A
// fragment Y[i % 4].  Operand registers: one set of X[0..6], two of X[7], two
// Y sets.  With half the MFMAs per K-step of the 256x256 kernel and the same
// B work per thread, every slot carries about one companion:
//   substep 0: wait for B(t+1) at slot 1, one byte-permute pair of its
//              transpose per slot over slots 1-16, B(t+2) loads every third
//              slot from 9 (into rows the transpose has finished with), the
//              B(t+1)^T writes into stage SN on the odd slots 17-31; reads of
//              substep 1's operands: X[a] at slot 4a + 4, X[7] at 18, Y[b] at
//              2 + 4b;
//   substep 1: wait for the A(t+1) copies and barrier at slot 4 (publishes
//              stage SN, frees stage S), A(t+2) copies at slots 5, 9, 13, 17,
//              reads of step t+1's substep-0 operands from stage SN: X[a] at
//              4a + 4, X[7] at 26, Y[b] at 6 + 4b.
// Ragged edges as in the other interleaved kernels.
#pragma once

#include <type_traits>

#include "gsr_interleave16.hpp"

namespace gsr {

struct Ilv16HCfg {
    static constexpr int BM = 128, BN = 256, BK = 64, WM = 2, WN = 2;
    static constexpr int NW = WM * WN, NT = kWave * NW;
    static constexpr int CH = BK / 8;
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    static constexpr int FM = WTM / 16, FN = WTN / 16;  // 4 (m) x 8 (n) blocks of 16x16
    static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
    static constexpr int B_REGION = 2 * A_BYTES;
    static constexpr int LDS_BYTES = 2 * (A_BYTES + B_BYTES);
    static constexpr int A_PER = A_BYTES / 1024 / NW;  // 4 copies per wave per step
    static constexpr int B_LOADS = 8;                  // one 8x8 block per thread
    static constexpr int SLOTS = FM * FN;              // MFMAs per substep
    static_assert((BK / 8) * (BN / 8) == NT, "one B block per thread");
    static_assert(A_PER == 4 && FM == 4 && FN == 8 && SLOTS == 32, "the slot plan below");
};

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_scale_relu_ilv16h_kernel(Problem p)
{
    using T = Ilv16HCfg;
    constexpr int BK = T::BK, CH = T::CH, FM = T::FM, FN = T::FN;

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

    // ---- descriptors that advance along K (as in the other interleaved kernels)
    uint64_t a_base = (uint64_t)(uintptr_t)p.A + ((uint64_t)m0 * K) * 2u;
    uint32_t a_recs = ((uint32_t)p.M * K - (uint32_t)m0 * K) * 2u;
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
    auto a_rsrc = [&](uint32_t k) { return (k < K) ? rsrc_of(a_base + (uint64_t)k * 2u, a_recs - k * 2u) : rsrc_of(a_base, 0u); };
    auto b_rsrc = [&](uint32_t k) {
        return (k < K) ? rsrc_of(b_base + (uint64_t)k * N * 2u, b_recs - k * N * 2u) : rsrc_of(b_base, 0u);
    };

    // ---- per-lane copy plan (that of the 256x256 16x16x32 kernel, 4 copies)
    // Copy i of this wave fills LDS chunk positions 64*(wave+4i) + lane: row
    // r = 8*wave + 32i + lane/8, logical chunk c0 ^ 4*(i & 1).
    const uint32_t c0 = ((uint32_t)lane & 7u) ^ ((uint32_t)lane >> 3) ^ (uint32_t)wave;
    const uint32_t arow = (8u * (uint32_t)wave + ((uint32_t)lane >> 3)) * K * 2u;
    uint32_t av0 = arow + 16u * c0, av1 = arow + 32u * K * 2u + 16u * (c0 ^ 4u);
    uint32_t kc0 = 8u * c0, kc1 = 8u * (c0 ^ 4u);
    const uint32_t a_istride = 64u * K * 2u;
    const uint32_t kb = (uint32_t)tid / (T::BN / 8), nb = (uint32_t)tid % (T::BN / 8);
    uint32_t b_off0 = ((uint32_t)n0 + nb * 8u < N) ? ((kb * 8u) * N + nb * 8u) * 2u : kOutOfRange;
    uint32_t bwq = (uint32_t)T::B_REGION + nb * 8u * (BK * 2) + (((kb ^ nb) & 7u) << 4);
    // Fragment addresses: B^T block a (rows wn*128 + 16a + l%16) for a = 0..3,
    // block a + 4 is 8 KiB further; the A block b (rows wm*64 + 16b + l%16)
    // has B^T block b's swizzle (the rows differ by a multiple of 64), so its
    // address is that one minus a wave-uniform distance; lane group g reads
    // chunk (g & 1) * 2 + g / 2 of the substep's four, and substep 1 flips
    // chunk bit 2.
    const uint32_t lrow = (uint32_t)lane & 15u, lq = (uint32_t)lane >> 4;
    const uint32_t lch = ((lq & 1u) << 1) | (lq >> 1);
    uint32_t xb[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const uint32_t rx = (uint32_t)wn * T::WTN + (uint32_t)a * 16u + lrow;
        xb[a] = (uint32_t)T::B_REGION + rx * (BK * 2) + ((lch ^ swz_a<CH>(rx)) << 4);
    }
    const uint32_t ydelta = (uint32_t)T::B_REGION + (uint32_t)((wn * T::WTN - wm * T::WTM) * (BK * 2));

    f32x4 acc[FN][FM];
#pragma unroll
    for (int a = 0; a < FN; ++a)
#pragma unroll
        for (int b = 0; b < FM; ++b) acc[a][b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    half8 X[FN - 1];  // B^T fragments 0..6, refilled one by one
    half8 X7[2];      // B^T fragment 7, one per substep parity
    half8 Y[2][FM];   // A fragments, one set per substep parity
    u32x4 breg[8];    // B block of a future step
    u32x4 bcol[8];    // its transpose

    auto copy_a = [&](int S, int i, uint32_t kleft, const i32x4& ra) {
        const uint32_t kc = (i & 1) ? kc1 : kc0;
        const uint32_t off = (kc < kleft) ? ((i & 1) ? av1 : av0) + (uint32_t)(i >> 1) * a_istride : kOutOfRange;
        copy16_to_lds(ra, off, lds0 + (uint32_t)(S * T::A_BYTES) + (uint32_t)(wave + i * T::NW) * 1024u);
    };
    auto b_voff = [&](int j) { return b_off0 + (uint32_t)j * N * 2u; };
    auto write_bt = [&](int S, int j) {
        *(u32x4*)(smem + S * T::B_BYTES + j * (BK * 2) + (bwq ^ ((uint32_t)j << 4))) = bcol[j];
    };
    auto read_x = [&](int S, int ks, int a) {
        const uint32_t off = xb[a & 3] ^ (ks ? 64u : 0u);
        const half8 v = __builtin_bit_cast(half8, *(const u32x4*)(smem + S * T::B_BYTES + (a >> 2) * (64 * BK * 2) + off));
        if (a == FN - 1) X7[ks] = v;
        else X[a] = v;
    };
    auto read_y = [&](int S, int ks, int b, half8& dst) {
        const uint32_t off = (xb[b] ^ (ks ? 64u : 0u)) - ydelta;
        dst = __builtin_bit_cast(half8, *(const u32x4*)(smem + S * T::A_BYTES + off));
    };
    // Reads of slot i of a substep, for the next substep (stage SR, substep
    // kr): X[a] (a < 7) at slot 4a + 4, X[7] at slot x7, Y[b] at y0 + 4b.
    auto reads = [&](int i, int SR, int kr, half8 (&ynext)[FM], int y0, int x7) {
        if ((i & 3) == 0 && i >= 4 && i <= 4 * (FN - 1)) read_x(SR, kr, (i >> 2) - 1);
        if (i == x7) read_x(SR, kr, FN - 1);
        if (i >= y0 && i < y0 + 4 * FM && ((i - y0) & 3) == 0) read_y(SR, kr, (i - y0) >> 2, ynext[(i - y0) >> 2]);
    };
    auto mma = [&](int i, int ks, const half8 (&ys)[FM]) {
        const int a = i >> 2;
        mfma16_inplace(acc[a][i & 3], a == FN - 1 ? X7[ks] : X[a], ys[i & 3]);
    };

    auto step = [&](auto stage_tag, int t) {
        constexpr int S = decltype(stage_tag)::value;
        constexpr int SN = S ^ 1;
        const uint32_t k2 = (uint32_t)(t + 2) * BK;
        asm volatile("" : "+v"(av0), "+v"(av1), "+v"(kc0), "+v"(kc1), "+v"(b_off0), "+v"(bwq), "+v"(xb[0]), "+v"(xb[1]),
                     "+v"(xb[2]), "+v"(xb[3]));
        // substep 0 (Y[0]); reads for substep 1 of this step
        {
            const i32x4 rb = b_rsrc(k2);
#pragma unroll
            for (int i = 0; i < T::SLOTS; ++i) {
                mma(i, 0, Y[0]);
                reads(i, S, 1, Y[1], 2, 18);
                if (i == 1) wait_vmcnt_b<T::A_PER>(breg);  // B(t+1) is in; A(t+1) copies may not be
                if (i >= 1 && i < 17) {
                    // one of the 16 byte-permute pairs (two permutes) per slot;
                    // rows 2e and 2e+1 of the block are consumed by slot 4e + 4
                    const int e = (i - 1) >> 2, d = (i - 1) & 3;
                    bcol[2 * d][e] = pack_lo(breg[2 * e][d], breg[2 * e + 1][d]);
                    bcol[2 * d + 1][e] = pack_hi(breg[2 * e][d], breg[2 * e + 1][d]);
                }
                if (i >= 9 && (i - 9) % 3 == 0 && (i - 9) / 3 < 8) breg[(i - 9) / 3] = load16(rb, b_voff((i - 9) / 3));
                if (i >= 17 && (i & 1)) write_bt(SN, (i - 17) >> 1);
                sched_fence();
            }
        }
        // substep 1 (Y[1]); after the barrier, reads for substep 0 of step t+1
        {
            const uint32_t kleft2 = (k2 < K) ? K - k2 : 0u;
            const i32x4 ra = a_rsrc(k2);
#pragma unroll
            for (int i = 0; i < T::SLOTS; ++i) {
                mma(i, 1, Y[1]);
                if (i == 4) {
                    wait_vmcnt<T::B_LOADS>();  // A(t+1) copies are in; B(t+2) loads may not be
                    lds_barrier();
                }
                if (i >= 4) reads(i, SN, 0, Y[0], 6, 26);
                if (i >= 5 && i < 21 && ((i - 5) & 3) == 0) copy_a(S, (i - 5) >> 2, kleft2, ra);
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
        for (int j = 0; j < 8; ++j) breg[j] = load16(rb, b_voff(j));
        wait_vmcnt_b<0>(breg);
        transpose8x8(breg, bcol);
#pragma unroll
        for (int j = 0; j < 8; ++j) write_bt(0, j);
        const i32x4 rb1 = b_rsrc((uint32_t)BK);
#pragma unroll
        for (int j = 0; j < 8; ++j) breg[j] = load16(rb1, b_voff(j));
        const uint32_t kleft1 = ((uint32_t)BK < K) ? K - (uint32_t)BK : 0u;
        const i32x4 ra1 = a_rsrc((uint32_t)BK);
#pragma unroll
        for (int i = 0; i < T::A_PER; ++i) copy_a(1, i, kleft1, ra1);
        lds_barrier();
        // substep-0 operands of step 0
#pragma unroll
        for (int a = 0; a < FN; ++a) read_x(0, 0, a);
#pragma unroll
        for (int b = 0; b < FM; ++b) read_y(0, 0, b, Y[0][b]);
    }

    for (int t = 0; t < ksteps; t += 2) {
        step(std::integral_constant<int, 0>{}, t);
        step(std::integral_constant<int, 1>{}, t + 1);
    }
    wait_vmcnt_b<0>(breg);

    // The MFMAs are opaque to the compiler's hazard tracking: give the last
    // of them the wait states a matrix result needs before it is read.
    asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15\n\ts_nop 15" ::: "memory");
    ilv16_epilogue_t<T>(p, acc, smem, m0, n0, wm, wn, wave);
}

}  // namespace gsr
