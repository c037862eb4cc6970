// gsr_interleave16c.hpp -- the B-through-LDS kernel of gsr_interleave16d.hpp
// with its copies moved to four waves of their own: the 128x256 tile
// (configuration 31, the copy-wave form of configuration 29) and the 128x128
// tile (configuration 32).
//
// In the B-through-LDS kernels every direct-to-LDS copy stalls the wave that
// issues it for 17-21 clocks of its matrix pipe: timing variants of the
// 128x256 kernel with the copies removed (same addresses, outputs not valid)
// ran the K-step in 1068 clocks instead of 1324, against 1024 for its MFMAs
// alone.  Here the workgroup has eight waves, two per SIMD: four MFMA waves
// with the data flow of configuration 29 minus its copies, and four copy
// waves that only issue the copies and wait for them.  The tile's
// accumulators take 128 AGPRs per MFMA wave, so both waves of a SIMD fit in
// its register file (128 VGPRs + 128 AGPRs each); the 256x256 tile, whose
// waves hold 256 AGPRs, has no room for this.
//
// LDS, stages, copy plans and fragments are those of configuration 29 (the
// copy plans with the copy wave's index in place of the wave's), and every
// MFMA pairs the same k, so the two give the same bits.  Per K-step t both
// kinds of wave pass one barrier b_t, which publishes stage t+1 and frees A
// stage t mod 2:
//   copy waves:  B(t+2) into B stage (t+2) mod 3 (free since b_{t-1}), wait
//                until only those copies are in flight (A(t+1) and B(t+1)
//                have landed), b_t, then A(t+2) into A stage t mod 2;
//   MFMA waves:  configuration 29's slot plan without its copies and waits:
//                substep 0 reads substep 1's operands, b_t at slot 4 of
//                substep 1, then step t+1's substep-0 reads.
// The prologue and the epilogue each hold one more barrier for all eight
// waves: copy waves land stage 0 before the first, and drain every copy
// before the epilogue's, after which they end.
//
// The 128x128 tile (configuration 32) runs the same MFMA waves on half the
// B columns, so its K-step is half as long while a copy takes as long to
// land: with the stages above, each A copy would have one short K-step from
// issue to the barrier that publishes it.  It keeps instead one ring of
// RING = 4 stages, each holding the A and the B tile of one K-step (128 KiB):
//   copy waves:  before the loop the copies of steps 0 .. 3; per K-step t,
//                wait until step t+1 has landed (the copies of t+2 and t+3
//                may still fly), b_t, then the copies of step t+4 into stage
//                t mod 4, which b_t freed;
//   MFMA waves:  the plan above with A and B both at stage t mod 4.
// A copy so has three K-steps to land.  On one MI355X this took the tile's
// time down by 17 % at the median of 60 shapes (up to 26 % at K >= 1536),
// with the same bits.  Its K-steps run one by one (the two-plus-three layout
// runs them in pairs, an odd count taking one step of zeros more).
#pragma once

#include <type_traits>
#include <utility>

#include "gsr_interleave16d.hpp"

namespace gsr {

// The 128x256 tile (configuration 31).
struct Ilv16CCfg {
    static constexpr int BM = 128, BN = 256, BK = 64, WM = 2, WN = 2;
    static constexpr int NW = WM * WN;                   // MFMA waves (0..3)
    static constexpr int NCW = 4;                        // copy waves (4..7)
    static constexpr int NT = kWave * (NW + NCW);        // 512 threads
    static constexpr int CH = BK / 8;
    static constexpr int WTM = BM / WM, WTN = BN / WN;   // 64 x 128 per MFMA wave
    static constexpr int FM = WTM / 16, FN = WTN / 16;   // 4 (m) x 8 (n) blocks of 16x16
    static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
    static constexpr int RING = 0;                       // two A stages, three B stages
    static constexpr int B_REGION = 2 * A_BYTES;
    static constexpr int ROWB = BN * 2;
    static constexpr int A_PER = A_BYTES / 1024 / NCW;   // 4 copies per copy wave per step
    static constexpr int B_PER = B_BYTES / 1024 / NCW;   // 8
    static constexpr int LDS_BYTES = 2 * A_BYTES + 3 * B_BYTES;  // 128 KiB
    static constexpr int SLOTS = FM * FN;                // 32 MFMAs per substep
    // configuration 29's read plan: X[7] at X7_0 / X7_1, Y[b] at Y0 + YS b
    static constexpr int X7_0 = Ilv16HDCfg::X7_0, X7_1 = Ilv16HDCfg::X7_1;
    static constexpr int Y0_0 = Ilv16HDCfg::Y0_0, Y0_1 = Ilv16HDCfg::Y0_1, YS = 4, BAR = Ilv16HDCfg::BAR;
};

// The 128x128 tile (configuration 32): four MFMA waves of 64x64, 4 (n) x 4
// (m) blocks of 16x16 each, 16 MFMAs per substep; B rows of 256 bytes (16
// chunks, the same fb16 swizzle); A and B tiles of 16 KiB, in a ring of four
// stages (128 KiB).
// Reads: the last B^T fragment at slots 1-2 of substep 0 and 2-3 of substep
// 1, the A^T fragments every second slot from 0 and from 1, the barrier at
// slot 1 of substep 1.
struct Ilv16QCCfg {
    static constexpr int BM = 128, BN = 128, BK = 64, WM = 2, WN = 2;
    static constexpr int NW = WM * WN;                   // MFMA waves (0..3)
    static constexpr int NCW = 4;                        // copy waves (4..7)
    static constexpr int NT = kWave * (NW + NCW);        // 512 threads
    static constexpr int CH = BK / 8;
    static constexpr int WTM = BM / WM, WTN = BN / WN;   // 64 x 64 per MFMA wave
    static constexpr int FM = WTM / 16, FN = WTN / 16;   // 4 (m) x 4 (n) blocks of 16x16
    static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
    static constexpr int RING = 4;                       // A and B stages, one ring
    static constexpr int B_REGION = RING * A_BYTES;
    static constexpr int ROWB = BN * 2;
    static constexpr int A_PER = A_BYTES / 1024 / NCW;   // 4 copies per copy wave per step
    static constexpr int B_PER = B_BYTES / 1024 / NCW;   // 4
    static constexpr int LDS_BYTES = RING * (A_BYTES + B_BYTES);  // 128 KiB
    static constexpr int SLOTS = FM * FN;                // 16 MFMAs per substep
    static constexpr int X7_0 = 1, X7_1 = 2;
    static constexpr int Y0_0 = 0, Y0_1 = 1, YS = 2, BAR = 1;
};

// f(integral_constant<int, I>) for each I of the sequence, in order
template <class F, int... I>
__device__ __forceinline__ void for_each_ic(F& f, std::integer_sequence<int, I...>)
{
    (f(std::integral_constant<int, I>{}), ...);
}

template <class T>
__global__ void __launch_bounds__(512) gemm_scale_relu_ilv16c_kernel(Problem p)
{
    constexpr int BK = T::BK, CH = T::CH, FM = T::FM, FN = T::FN;
    constexpr uint32_t CPR = T::BN / 8, RPK = 1024 / T::ROWB;  // chunks per B row, B rows per 1 KiB copy
    static_assert(BK == 64 && (T::BN == 256 || T::BN == 128) && T::WTN == T::BN / 2 && T::BM == 128,
                  "the copy and read plans below");
    static_assert(T::A_PER == 4 && T::NW == 4 && T::NCW == 4, "the copy plans below");
    static_assert(T::LDS_BYTES <= 163840, "LDS budget of one workgroup on gfx950");
    static_assert(T::RING == 0 || (T::RING >= 3 && (T::RING - 1) * (T::A_PER + T::B_PER) < 64),
                  "a ring of three stages or more; the copies in flight fit the vmcnt field");
    static_assert(T::RING != 0 || T::B_BYTES + 32 * T::ROWB + 4 * T::ROWB < 65536, "B read offsets fit the immediate field");
    static_assert(FM >= T::BAR && T::Y0_1 >= T::BAR && T::X7_1 >= T::BAR, "reads of the new stages follow the barrier");
    static_assert(T::X7_0 + 1 < FM * (FN - 1) && T::Y0_0 + T::YS * (FM - 1) < T::SLOTS && T::Y0_1 + T::YS * (FM - 1) < T::SLOTS,
                  "operands of the next substep are read within this one");

    __shared__ __attribute__((aligned(1024))) uint8_t smem[T::LDS_BYTES];  // A stages, then B stages

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    int tm, tn;
    tile_of(blockIdx.x, gridDim.x, p, tm, tn);
    const int m0 = tm * T::BM, n0 = tn * T::BN;
    const uint32_t K = (uint32_t)p.K, N = (uint32_t)p.N;
    const uint32_t lds0 = lds_address(smem);
    // K-steps: the two-plus-three layout runs them in pairs (an odd count
    // takes one more step of zeros), the ring one by one
    const int ksteps = T::RING ? ((int)K + BK - 1) / BK : (((int)K + BK - 1) / BK + 1) & ~1;

    if (wave >= T::NW) {
        // ======================= copy waves =================================
        const uint32_t cw = (uint32_t)(wave - T::NW);
        const uint64_t a_base = (uint64_t)(uintptr_t)p.A + ((uint64_t)m0 * K) * 2u;
        const uint32_t a_recs = ((uint32_t)p.M * K - (uint32_t)m0 * K) * 2u;
        const uint64_t b_base = (uint64_t)(uintptr_t)p.B + (uint64_t)n0 * 2u;
        const uint32_t b_recs = (K * N - (uint32_t)n0) * 2u;
        auto rsrc_of = [](uint64_t base, uint32_t recs) {
            i32x4 r;
            r[0] = (int)(uint32_t)base;
            r[1] = (int)((uint32_t)(base >> 32) & 0xffffu);
            r[2] = (int)recs;
            r[3] = 0x00020000;
            return r;
        };
        // positioned at column k of A / row k of B; from k = K on they cover
        // no bytes, so every copy through them writes zeros
        auto a_rsrc = [&](uint32_t k) { return (k < K) ? rsrc_of(a_base + (uint64_t)k * 2u, a_recs - k * 2u) : rsrc_of(a_base, 0u); };
        auto b_rsrc = [&](uint32_t k) {
            return (k < K) ? rsrc_of(b_base + (uint64_t)k * N * 2u, b_recs - k * N * 2u) : rsrc_of(b_base, 0u);
        };
        // A: copy i fills the 1 KiB block cw + 4i (rows 8 cw + 32 i + lane / 8)
        const uint32_t c0 = ((uint32_t)lane & 7u) ^ ((uint32_t)lane >> 3) ^ cw;
        const uint32_t arow = (8u * cw + ((uint32_t)lane >> 3)) * K * 2u;
        const uint32_t av0 = arow + 16u * c0, av1 = arow + 32u * K * 2u + 16u * (c0 ^ 4u);
        const uint32_t kc0 = 8u * c0, kc1 = 8u * (c0 ^ 4u);
        const uint32_t a_istride = 64u * K * 2u;
        // B: copy i fills chunk positions 64 (cw + 4i) + lane of the stage:
        // row k = RPK (cw + 4i) + lane / CPR, logical chunk
        // (lane % CPR) ^ fb16(k) (fb16 touches chunk bits 1-3 only)
        uint32_t b_voff[T::B_PER];
#pragma unroll
        for (int i = 0; i < T::B_PER; ++i) {
            const uint32_t k = RPK * (cw + 4u * (uint32_t)i) + (uint32_t)lane / CPR;
            const uint32_t c = ((uint32_t)lane & (CPR - 1u)) ^ fb16(k);
            b_voff[i] = ((uint32_t)n0 + 8u * c < N) ? (k * N + 8u * c) * 2u : kOutOfRange;
        }
        auto copy_a = [&](uint32_t stage, uint32_t k) {
            const uint32_t kleft = (k < K) ? K - k : 0u;
            const i32x4 ra = a_rsrc(k);
#pragma unroll
            for (int i = 0; i < T::A_PER; ++i) {
                const uint32_t kc = (i & 1) ? kc1 : kc0;
                const uint32_t off = (kc < kleft) ? ((i & 1) ? av1 : av0) + (uint32_t)(i >> 1) * a_istride : kOutOfRange;
                copy16_to_lds(ra, off, lds0 + stage * (uint32_t)T::A_BYTES + (cw + (uint32_t)i * T::NCW) * 1024u);
            }
        };
        auto copy_b = [&](uint32_t stage, uint32_t k) {
            const i32x4 rb = b_rsrc(k);
#pragma unroll
            for (int i = 0; i < T::B_PER; ++i)
                copy16_to_lds(rb, b_voff[i], lds0 + (uint32_t)T::B_REGION + stage * (uint32_t)T::B_BYTES + (cw + (uint32_t)i * T::NCW) * 1024u);
        };
        if constexpr (T::RING == 0) {
            copy_a(0, 0);
            copy_b(0, 0);
            copy_a(1, (uint32_t)BK);
            copy_b(1, (uint32_t)BK);
            wait_vmcnt<T::A_PER + T::B_PER>();  // stage 0 has landed
            lds_barrier();
            for (int t = 0; t < ksteps; ++t) {
                const uint32_t k2 = (uint32_t)(t + 2) * BK;
                copy_b((uint32_t)((t + 2) % 3), k2);
                wait_vmcnt<T::B_PER>();  // A(t+1), B(t+1) have landed; B(t+2) may not have
                lds_barrier();           // b_t
                copy_a((uint32_t)(t & 1), k2);
            }
        } else {
            // one ring of RING stages, each holding the A and the B tile of
            // one K-step: K-step s goes to stage s mod RING, issued RING - 1
            // K-steps before the barrier that publishes it
            constexpr int PER = T::A_PER + T::B_PER;
#pragma unroll
            for (int s = 0; s < T::RING; ++s) {
                copy_a((uint32_t)s, (uint32_t)(s * BK));
                copy_b((uint32_t)s, (uint32_t)(s * BK));
            }
            wait_vmcnt<(T::RING - 1) * PER>();  // stage 0 has landed
            lds_barrier();
            for (int t = 0; t < ksteps; ++t) {
                wait_vmcnt<(T::RING - 2) * PER>();  // step t+1 has landed; t+2 .. t+RING-1 may not have
                lds_barrier();                      // b_t: frees stage t mod RING
                const uint32_t s = (uint32_t)(t % T::RING), k = (uint32_t)(t + T::RING) * BK;
                copy_a(s, k);
                copy_b(s, k);
            }
        }
        wait_vmcnt<0>();  // no copy may land in LDS once the epilogue reuses it
        lds_barrier();    // the epilogue's
        return;
    }

    // ========================== MFMA waves ==================================
    const int wm = wave / T::WN, wn = wave % T::WN;
    const uint32_t lrow = (uint32_t)lane & 15u, lq = (uint32_t)lane >> 4;
    const uint32_t lch = ((lq & 1u) << 1) | (lq >> 1);
    // A^T fragment b, substep 0 (substep 1: byte offset ^ 64)
    uint32_t yb[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const uint32_t ry = (uint32_t)wm * T::WTM + (uint32_t)b * 16u + lrow;
        yb[b] = ry * (BK * 2) + ((lch ^ swz_a<CH>(ry)) << 4);
    }
    // B^T fragment a by transpose reads, B stage 0 (stage 1 rides in the
    // immediate, stage 2 is added when read): logical chunk
    // (WTN / 8) wn + 2a + q / 2 of row 8 lch(g) + e sits at physical chunk
    // (that) ^ fb16(row)
    uint32_t xa[FN];
    {
        const uint32_t e = lrow >> 2, q = lrow & 3u;
        const uint32_t krow0 = 8u * lch + e;
        const uint32_t f = fb16(krow0);
        if constexpr (T::WTN == 128) {  // the XOR stays inside the wave's 16 chunks
            const uint32_t base = (uint32_t)T::B_REGION + krow0 * T::ROWB + (16u * (uint32_t)wn + (q >> 1)) * 16u + (q & 1u) * 8u;
#pragma unroll
            for (int a = 0; a < FN; ++a) xa[a] = base + ((((uint32_t)a) ^ (f >> 1)) << 5);
        } else {
#pragma unroll
            for (int a = 0; a < FN; ++a) {
                const uint32_t chunk = ((uint32_t)(T::WTN / 8) * (uint32_t)wn + 2u * (uint32_t)a + (q >> 1)) ^ f;
                xa[a] = (uint32_t)T::B_REGION + krow0 * T::ROWB + (chunk << 4) + (q & 1u) * 8u;
            }
        }
    }

    f32x4 acc[FN][FM];
#pragma unroll
    for (int a = 0; a < FN; ++a)
#pragma unroll
        for (int b = 0; b < FM; ++b) acc[a][b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    half8 X[FN - 1];  // B^T fragments 0..6, refilled one by one
    half8 X7[2];      // B^T fragment 7, one per substep parity
    half8 Y[2][FM];   // A^T fragments, one set per substep parity
    v4i16 xlo[FN];    // first half of a B^T fragment, waiting for its second

    auto read_xh = [&](int S, int ks, int a, int rd) {
        // the ring's stages ride in the immediate; of the three B stages of
        // the two-plus-three layout only stage 1 does
        const uint32_t off = (uint32_t)((T::RING ? S * T::B_BYTES : (S == 1 ? T::B_BYTES : 0)) + ks * 32 * T::ROWB + rd * 4 * T::ROWB);
        const uint32_t addr = (!T::RING && S == 2) ? xa[a] + 2u * (uint32_t)T::B_BYTES : xa[a];
        const v4i16 h = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(smem + addr + off));
        if (rd == 0) {
            xlo[a] = h;
        } else {
            const half8 v = __builtin_bit_cast(half8, __builtin_shufflevector(xlo[a], h, 0, 1, 2, 3, 4, 5, 6, 7));
            if (a == FN - 1) X7[ks] = v;
            else X[a] = v;
        }
    };
    auto read_y = [&](int S, int ks, int b, half8& dst) {
        dst = __builtin_bit_cast(half8, *(const u32x4*)(smem + S * T::A_BYTES + (yb[b] ^ (ks ? 64u : 0u))));
    };
    // reads of slot i for the next substep: X[a] (a < FN - 1) at slots
    // FM (a + 1) and FM (a + 1) + 1, the last X at x7 and x7 + 1, Y[b] at
    // y0 + YS b
    auto reads = [&](int i, int SR, int BR, int kr, half8 (&ynext)[FM], int y0, int x7) {
        constexpr int YS = T::YS;
        if (i >= FM && i <= FM * (FN - 1) + 1 && (i % FM) < 2) read_xh(BR, kr, i / FM - 1, i % FM);
        if (i == x7 || i == x7 + 1) read_xh(BR, kr, FN - 1, i - x7);
        if (i >= y0 && i < y0 + YS * FM && ((i - y0) % YS) == 0) read_y(SR, kr, (i - y0) / YS, ynext[(i - y0) / YS]);
    };
    auto mma = [&](int i, int ks, const half8 (&ys)[FM]) {
        const int a = i / FM;
        mfma16_inplace(acc[a][i % FM], a == FN - 1 ? X7[ks] : X[a], ys[i % FM]);
    };
    auto step = [&](auto a_tag, auto b_tag) {
        constexpr int SA = decltype(a_tag)::value, SB = decltype(b_tag)::value;
        constexpr int SAN = T::RING ? (SA + 1) % T::RING : SA ^ 1, SBN = T::RING ? (SB + 1) % T::RING : (SB + 1) % 3;
#pragma unroll
        for (int i = 0; i < T::SLOTS; ++i) {
            mma(i, 0, Y[0]);
            reads(i, SA, SB, 1, Y[1], T::Y0_0, T::X7_0);
            sched_fence();
        }
#pragma unroll
        for (int i = 0; i < T::SLOTS; ++i) {
            mma(i, 1, Y[1]);
            if (i == T::BAR) lds_barrier();  // b_t: stage t+1 published, A stage SA freed
            if (i >= T::BAR) reads(i, SAN, SBN, 0, Y[0], T::Y0_1, T::X7_1);
            sched_fence();
        }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;

    lds_barrier();  // stage 0 has landed
#pragma unroll
    for (int a = 0; a < FN; ++a) {
        read_xh(0, 0, a, 0);
        read_xh(0, 0, a, 1);
    }
#pragma unroll
    for (int b = 0; b < FM; ++b) read_y(0, 0, b, Y[0][b]);

    int t = 0;
    if constexpr (T::RING == 0) {
        for (; t + 6 <= ksteps; t += 6) {
            step(I0{}, I0{});
            step(I1{}, I1{});
            step(I0{}, I2{});
            step(I1{}, I0{});
            step(I0{}, I1{});
            step(I1{}, I2{});
        }
        if (t + 2 <= ksteps) {
            step(I0{}, I0{});
            step(I1{}, I1{});
            t += 2;
        }
        if (t + 2 <= ksteps) {
            step(I0{}, I2{});
            step(I1{}, I0{});
        }
    } else {
        auto ring_step = [&](auto s_tag) { step(s_tag, s_tag); };
        for (; t + T::RING <= ksteps; t += T::RING)
            for_each_ic(ring_step, std::make_integer_sequence<int, T::RING>{});
        // the rest: fewer than RING steps, from stage 0
        auto ring_tail = [&](auto s_tag) {
            if (t < ksteps) {
                step(s_tag, s_tag);
                ++t;
            }
        };
        for_each_ic(ring_tail, std::make_integer_sequence<int, T::RING - 1>{});
    }

    // The MFMAs above are opaque to the compiler's hazard tracking: give the
    // last of them the wait states a matrix result needs before other
    // instructions read it (64, well above the 16x16x32 requirement).
    asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15\n\ts_nop 15" ::: "memory");
    ilv16_epilogue_t<T>(p, acc, smem, m0, n0, wm, wn, wave);
}

}  // namespace gsr
