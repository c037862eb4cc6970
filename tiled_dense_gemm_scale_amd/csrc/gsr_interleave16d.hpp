// gsr_interleave16d.hpp -- the explicitly interleaved kernels on the
// 16x16x32 fp16 MFMA with both operands copied global -> LDS by the buffer
// unit: 256x256 tiles (configuration 28) and 128x256 tiles (configuration 29).
//
// Waves, accumulators, A path, A^T fragments, launch order and epilogue are
// those of the register-transpose kernel in gsr_interleave16.hpp (256x256;
// the 128x256 tile is the same at half the height: four waves of 64x128,
// 8 (n) x 4 (m) accumulator blocks each).  What changes is B: instead of
// loading an 8x8 block per thread into registers, transposing it with byte
// permutes and writing B^T rows to LDS, the buffer unit copies B straight
// into LDS as it is stored (64 k-rows of 256 n, 512 bytes each), and each
// B^T fragment is assembled from two gfx950 transpose reads
// (ds_read_b64_tr_b16), each handing a lane four k-consecutive values of one
// column.  Timing variants of the register-transpose 256x256 kernel with
// single parts of a K-step removed (same addresses, outputs not valid) put
// the B register path -- 8 global loads, 32 permutes and 8 LDS writes per
// wave per step -- at about a quarter of the kernel's time at 16384^3, more
// than the A copies (8 %) or all operand reads (9 %); the copies and
// transpose reads that replace it move the same bytes through LDS.  Both
// tiles keep B 256 wide, so every wave owns 128 columns and the B copy plan,
// swizzle and reads are one code for both.
//
// B layout in a stage: row k (0..63) at k * 512, its 16-byte chunk c at
// physical chunk c ^ fb(k), fb(k) = 2 * ((k mod 4) + 4 * s((k / 8) mod 4)),
// s(c) = (c ^ c / 2) mod 2.  A transpose read of fragment a gives 16-lane
// group g the rows 8 * lch(g) + 4 rd + 0..3 of its substep (lch as for the
// A^T fragments, so both operands pair the same k) and 32 bytes of each; the
// eight rows that the LDS serves in one cycle (lane groups 0 and 1, or 0 and
// 2, either way) then sit on eight distinct 32-byte bank slots.
//
// LDS: A0 | A1 | B0 | B1 | B2 (160 KiB at 256x256, 128 KiB at 128x256).
// Step t reads A stage t mod 2 and B stage t mod 3; the loop is unrolled
// over six steps so every stage offset is a constant.  A third B stage lets
// the copies of a step be spread over both substeps of the step before the
// one that publishes them: timing variants of the 256x256 kernel with all 16
// copies of a step packed into one substep after the barrier ran 5-6 %
// slower than with the same copies spread over that substep, and with only
// A's or B's copies removed each set still cost about 13 %, so the copies
// are given the whole K-step.
//
// A K-step is two 32-deep substeps of FM x FN MFMAs (FN = 8 B^T fragments
// of 16 columns, FM = 8 or 4 A^T fragments of 16 rows); slot i of a substep
// multiplies X[i / FM] with Y[i % FM].  Companions of step t (A stage
// SA = t mod 2, B stage SB = t mod 3), slots for 256x256 / 128x256:
//   substep 0: reads of substep 1's operands (X[a] as two transpose reads at
//              slots FM (a + 1) and FM (a + 1) + 1, X[7] at 44, 45 / 18, 19,
//              Y[b] every fourth slot from 2); the eight copies of B(t+2)
//              into B stage (t+2) mod 3, freed at step t-1's barrier, every
//              eighth slot from 4 / every fourth slot from 3;
//   substep 1, slot 6 / 4: wait for the A(t+1) and B(t+1) copies, barrier
//              (publishes step t+1, frees A stage SA); then the copies of
//              A(t+2) into A stage SA (8 every seventh slot from 8 / 4 every
//              fourth slot from 5), and the reads of step t+1's substep-0
//              operands (X[a] as in substep 0, X[7] at 60, 61 / 26, 27, Y[b]
//              every fourth slot from 10 / 6).
#pragma once

#include <type_traits>

#include "gsr_interleave16.hpp"

namespace gsr {

// The 256x256 tile (configuration 28) and its slot plan.
struct Ilv16DCfg : Ilv16Cfg {
    static constexpr int ROWB = BN * 2;                 // 512-byte B rows
    static constexpr int B_PER = B_BYTES / 1024 / NW;   // 8 copies per wave per step
    static constexpr int B_STAGES = 3;
    static constexpr int LDS_BYTES = 2 * A_BYTES + B_STAGES * B_BYTES;  // 160 KiB
    static constexpr int SLOTS = FM * FN;               // 64 MFMAs per substep
    static constexpr int X7_0 = 44, X7_1 = 60;          // X[7] reads in substeps 0 and 1
    static constexpr int Y0_0 = 2, Y0_1 = 10;           // first Y read in substeps 0 and 1
    static constexpr int BAR = 6;                       // wait + barrier slot of substep 1
    static constexpr int BC0 = 4, BCD = 8;              // B copies in substep 0: first slot, stride
    static constexpr int AC0 = 8, ACD = 7;              // A copies in substep 1: first slot, stride
};

// The 128x256 tile (configuration 29; gsr_interleave16c.hpp runs the same
// plan with its copies on separate waves, configuration 31): four waves of
// 64x128, 8 (n) x 4 (m) blocks of 16x16 per wave, 32 MFMAs per substep; A
// stages of 16 KiB, B stages as above (2 x 16 + 3 x 32 = 128 KiB).
struct Ilv16HDCfg {
    static constexpr int BM = 128, BN = 256, BK = 64, WM = 2, WN = 2;
    static constexpr int NW = WM * WN, NT = kWave * NW;
    static constexpr int CH = BK / 8;
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    static constexpr int FM = WTM / 16, FN = WTN / 16;  // 4 (m) x 8 (n) blocks of 16x16
    static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
    static constexpr int B_REGION = 2 * A_BYTES;
    static constexpr int ROWB = BN * 2;
    static constexpr int A_PER = A_BYTES / 1024 / NW;   // 4 copies per wave per step
    static constexpr int B_PER = B_BYTES / 1024 / NW;   // 8
    static constexpr int B_STAGES = 3;
    static constexpr int LDS_BYTES = 2 * A_BYTES + B_STAGES * B_BYTES;  // 128 KiB
    static constexpr int SLOTS = FM * FN;               // 32 MFMAs per substep
    static constexpr int X7_0 = 18, X7_1 = 26;
    static constexpr int Y0_0 = 2, Y0_1 = 6;
    static constexpr int BAR = 4;
    static constexpr int BC0 = 3, BCD = 4;
    static constexpr int AC0 = 5, ACD = 4;
};

// Physical-chunk mask of B row k (bits 1..3 of the chunk index only).
__device__ __forceinline__ uint32_t fb16(uint32_t k)
{
    const uint32_t c = (k >> 3) & 3u;
    return ((k & 3u) + (((c ^ (c >> 1)) & 1u) << 2)) << 1;
}

template <class T>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_scale_relu_ilv16d_kernel(Problem p)
{
    constexpr int BK = T::BK, CH = T::CH, FM = T::FM, FN = T::FN;
    static_assert(BK == 64 && T::BN == 256 && T::WTN == 128, "the B swizzle and read plan assume 64 rows of 32 chunks");
    static_assert(T::LDS_BYTES <= 163840, "LDS budget of one workgroup on gfx950");
    // ds_read offsets are 16 bits: B stages 0 and 1, substep and read ride in
    // them (stage 2 has a base register of its own)
    static_assert(T::B_BYTES + 32 * T::ROWB + 4 * T::ROWB < 65536, "B read offsets fit the immediate field");
    // the slot plan: every copy inside its substep, the barrier before any
    // read of the stages it publishes, X[7] and the Y reads in free registers
    // and early enough for their first MFMA
    static_assert(T::SLOTS == FM * FN && T::B_PER == 8 && FN == 8, "eight B^T fragments, eight B copies");
    static_assert(T::BC0 + T::BCD * (T::B_PER - 1) < T::SLOTS, "B copies fit substep 0");
    static_assert(T::AC0 > T::BAR && T::AC0 + T::ACD * (T::A_PER - 1) < T::SLOTS, "A copies follow the barrier");
    static_assert(T::Y0_1 >= T::BAR && T::X7_1 >= T::BAR && FM >= T::BAR, "reads of the new stages follow the barrier");
    static_assert(T::X7_0 + 1 < FM * (FN - 1) && T::Y0_0 + 4 * (FM - 1) < T::SLOTS && T::Y0_1 + 4 * (FM - 1) < T::SLOTS,
                  "operands of the next substep are read within this one");

    __shared__ __attribute__((aligned(1024))) uint8_t smem[T::LDS_BYTES];  // A0 | A1 | B0 | B1 | B2

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / T::WN, wn = wave % T::WN;

    int tm, tn;
    tile_of(blockIdx.x, gridDim.x, p, tm, tn);
    const int m0 = tm * T::BM, n0 = tn * T::BN;
    const uint32_t K = (uint32_t)p.K, N = (uint32_t)p.N;
    const uint32_t lds0 = lds_address(smem);

    // ---- descriptors that advance along K (as in the register-transpose kernel)
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
    // Positioned at column k of A / row k of B; from k = K on they cover no
    // bytes, so every copy through them writes zeros (rows of B past K fall
    // past the records as well).
    auto a_rsrc = [&](uint32_t k) { return (k < K) ? rsrc_of(a_base + (uint64_t)k * 2u, a_recs - k * 2u) : rsrc_of(a_base, 0u); };
    auto b_rsrc = [&](uint32_t k) {
        return (k < K) ? rsrc_of(b_base + (uint64_t)k * N * 2u, b_recs - k * N * 2u) : rsrc_of(b_base, 0u);
    };

    // ---- A copy plan (as in the register-transpose kernel) ------------------
    const uint32_t c0 = ((uint32_t)lane & 7u) ^ ((uint32_t)lane >> 3) ^ (uint32_t)wave;
    const uint32_t arow = (8u * (uint32_t)wave + ((uint32_t)lane >> 3)) * K * 2u;
    uint32_t av0 = arow + 16u * c0, av1 = arow + 32u * K * 2u + 16u * (c0 ^ 4u);
    uint32_t kc0 = 8u * c0, kc1 = 8u * (c0 ^ 4u);
    const uint32_t a_istride = 64u * K * 2u;

    // ---- B copy plan --------------------------------------------------------
    // Copy i of this wave fills B chunk positions P = 64 (wave + 4i) + lane:
    // row k = P / 32 = 2 wave + 8 i + lane / 32, physical chunk lane % 32,
    // logical chunk c = (lane % 32) ^ fb16(k), i.e. columns n0 + 8c .. +7.
    // Columns past N read as zero (N is a multiple of 8 on this path, so a
    // chunk is wholly in or out); rows past K fall past the descriptor.
    uint32_t b_voff[T::B_PER];
#pragma unroll
    for (int i = 0; i < T::B_PER; ++i) {
        const uint32_t k = 2u * (uint32_t)wave + 8u * (uint32_t)i + ((uint32_t)lane >> 5);
        const uint32_t c = ((uint32_t)lane & 31u) ^ fb16(k);
        b_voff[i] = ((uint32_t)n0 + 8u * c < N) ? (k * N + 8u * c) * 2u : kOutOfRange;
    }

    // ---- fragment addresses -------------------------------------------------
    // Lane group g = l / 16 takes k-group chunk lch(g) = (g & 1) * 2 + g / 2
    // of its substep for both operands (the A^T layout needs that order to be
    // free of bank conflicts).
    const uint32_t lrow = (uint32_t)lane & 15u, lq = (uint32_t)lane >> 4;
    const uint32_t lch = ((lq & 1u) << 1) | (lq >> 1);
    // A^T fragment b (0..3; b + 4 is 64 rows = 8 KiB further, same swizzle),
    // substep 0; substep 1 flips chunk bit 2 (byte offset ^ 64).
    uint32_t yb[2][4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const uint32_t ry = (uint32_t)wm * T::WTM + (uint32_t)b * 16u + lrow;
        yb[0][b] = ry * (BK * 2) + ((lch ^ swz_a<CH>(ry)) << 4);
        yb[1][b] = yb[0][b] ^ 64u;
    }
    // B^T fragment a (0..7) by transpose reads: in 16-lane group g, lane
    // i = 4e + q supplies the address of row 8 lch(g) + e (+ 4 for the second
    // read, + 32 for substep 1) and columns 16a + 4q .. +3 of this wave's 128;
    // fb16 of every such row is that of row 8 lch(g) + e.
    // xa: B stages 0 and 1 (the stage offset rides in the immediate), xa2:
    // B stage 2.
    uint32_t xa[FN], xa2[FN];
    {
        const uint32_t e = lrow >> 2, q = lrow & 3u;
        const uint32_t krow0 = 8u * lch + e;
        const uint32_t h = fb16(krow0) >> 1;
        const uint32_t base = (uint32_t)T::B_REGION + krow0 * T::ROWB + (16u * (uint32_t)wn + (q >> 1)) * 16u + (q & 1u) * 8u;
#pragma unroll
        for (int a = 0; a < FN; ++a) {
            xa[a] = base + ((((uint32_t)a) ^ h) << 5);
            xa2[a] = xa[a] + 2u * (uint32_t)T::B_BYTES;
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

    auto copy_a = [&](int S, int i, uint32_t kleft, const i32x4& ra) {
        const uint32_t kc = (i & 1) ? kc1 : kc0;
        const uint32_t off = (kc < kleft) ? ((i & 1) ? av1 : av0) + (uint32_t)(i >> 1) * a_istride : kOutOfRange;
        copy16_to_lds(ra, off, lds0 + (uint32_t)(S * T::A_BYTES) + (uint32_t)(wave + i * T::NW) * 1024u);
    };
    auto copy_b = [&](int S, int i, const i32x4& rb) {
        copy16_to_lds(rb, b_voff[i], lds0 + (uint32_t)(T::B_REGION + S * T::B_BYTES) + (uint32_t)(wave + i * T::NW) * 1024u);
    };
    // half rd (0: k 0..3 of the lane's 8, 1: k 4..7) of B^T fragment a,
    // substep ks, B stage S
    auto read_xh = [&](int S, int ks, int a, int rd) {
        const uint32_t off = (uint32_t)((S == 1 ? T::B_BYTES : 0) + ks * 32 * T::ROWB + rd * 4 * T::ROWB);
        const v4i16 h = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(smem + (S == 2 ? xa2[a] : xa[a]) + off));
        if (rd == 0) {
            xlo[a] = h;
        } else {
            const half8 v = __builtin_bit_cast(half8, __builtin_shufflevector(xlo[a], h, 0, 1, 2, 3, 4, 5, 6, 7));
            if (a == FN - 1) X7[ks] = v;
            else X[a] = v;
        }
    };
    auto read_y = [&](int S, int ks, int b, half8& dst) {
        dst = __builtin_bit_cast(half8, *(const u32x4*)(smem + S * T::A_BYTES + (b >> 2) * (64 * BK * 2) + yb[ks][b & 3]));
    };
    // The reads of slot i of a substep, all for the next substep (A stage SR,
    // B stage BR, substep kr): X[a] (a < 7) at slots FM (a + 1) and
    // FM (a + 1) + 1, as soon as its last MFMA here has issued; X[7] (into
    // the other X7 register) at x7 and x7 + 1; Y[b] at slot y0 + 4b.
    auto reads = [&](int i, int SR, int BR, int kr, half8 (&ynext)[FM], int y0, int x7) {
        if (i >= FM && i <= FM * (FN - 1) + 1 && (i % FM) < 2) read_xh(BR, kr, i / FM - 1, i % FM);
        if (i == x7 || i == x7 + 1) read_xh(BR, kr, FN - 1, i - x7);
        if (i >= y0 && i < y0 + 4 * FM && ((i - y0) & 3) == 0) read_y(SR, kr, (i - y0) >> 2, ynext[(i - y0) >> 2]);
    };
    // slot i multiplies B^T fragment X[i / FM] with A^T fragment Y[i % FM]
    auto mma = [&](int i, int ks, const half8 (&ys)[FM]) {
        const int a = i / FM;
        mfma16_inplace(acc[a][i % FM], a == FN - 1 ? X7[ks] : X[a], ys[i % FM]);
    };

    // One K-step: A stage SA = t mod 2, B stage SB = t mod 3.
    auto step = [&](auto a_tag, auto b_tag, int t) {
        constexpr int SA = decltype(a_tag)::value, SB = decltype(b_tag)::value;
        constexpr int SAN = SA ^ 1, SBN = (SB + 1) % 3, SB2 = (SB + 2) % 3;
        const uint32_t k2 = (uint32_t)(t + 2) * BK;
        // Opaque to the optimiser from here on, so per-copy offsets are formed
        // where they are used instead of being hoisted into live registers.
        asm volatile("" : "+v"(av0), "+v"(av1), "+v"(kc0), "+v"(kc1));
        // substep 0 (Y[0]); reads for substep 1 of this step; B(t+2) copies
        {
            const i32x4 rb = b_rsrc(k2);
#pragma unroll
            for (int i = 0; i < T::SLOTS; ++i) {
                mma(i, 0, Y[0]);
                reads(i, SA, SB, 1, Y[1], T::Y0_0, T::X7_0);
                if (i >= T::BC0 && (i - T::BC0) % T::BCD == 0) copy_b(SB2, (i - T::BC0) / T::BCD, rb);
                sched_fence();
            }
        }
        // substep 1 (Y[1]); after the barrier, the A(t+2) copies into the
        // freed A stage and the reads for substep 0 of step t+1
        {
            const uint32_t kleft2 = (k2 < K) ? K - k2 : 0u;
            const i32x4 ra = a_rsrc(k2);
#pragma unroll
            for (int i = 0; i < T::SLOTS; ++i) {
                mma(i, 1, Y[1]);
                if (i == T::BAR) {
                    wait_vmcnt<T::B_PER>();  // A(t+1), B(t+1) are in; B(t+2) may not be
                    lds_barrier();
                }
                if (i >= T::BAR) reads(i, SAN, SBN, 0, Y[0], T::Y0_1, T::X7_1);
                if (i >= T::AC0 && (i - T::AC0) % T::ACD == 0 && (i - T::AC0) / T::ACD < T::A_PER)
                    copy_a(SA, (i - T::AC0) / T::ACD, kleft2, ra);
                sched_fence();
            }
        }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;

    // ---- prologue: A(0), B(0) in stage 0, A(1), B(1) in stage 1 -------------
    const int ksteps = (((int)K + BK - 1) / BK + 1) & ~1;  // even
    {
        const i32x4 ra0 = a_rsrc(0), rb0 = b_rsrc(0);
#pragma unroll
        for (int i = 0; i < T::A_PER; ++i) copy_a(0, i, K, ra0);
#pragma unroll
        for (int i = 0; i < T::B_PER; ++i) copy_b(0, i, rb0);
        const uint32_t kleft1 = ((uint32_t)BK < K) ? K - (uint32_t)BK : 0u;
        const i32x4 ra1 = a_rsrc((uint32_t)BK), rb1 = b_rsrc((uint32_t)BK);
#pragma unroll
        for (int i = 0; i < T::A_PER; ++i) copy_a(1, i, kleft1, ra1);
#pragma unroll
        for (int i = 0; i < T::B_PER; ++i) copy_b(1, i, rb1);
        wait_vmcnt<T::A_PER + T::B_PER>();  // stage 0's copies are in
        lds_barrier();
        // substep-0 operands of step 0
#pragma unroll
        for (int a = 0; a < FN; ++a) {
            read_xh(0, 0, a, 0);
            read_xh(0, 0, a, 1);
        }
#pragma unroll
        for (int b = 0; b < FM; ++b) read_y(0, 0, b, Y[0][b]);
    }

    // six steps per iteration (A stages repeat every two, B stages every
    // three), then two or four more: ksteps is even
    int t = 0;
    for (; t + 6 <= ksteps; t += 6) {
        step(I0{}, I0{}, t);
        step(I1{}, I1{}, t + 1);
        step(I0{}, I2{}, t + 2);
        step(I1{}, I0{}, t + 3);
        step(I0{}, I1{}, t + 4);
        step(I1{}, I2{}, t + 5);
    }
    if (t + 2 <= ksteps) {
        step(I0{}, I0{}, t);
        step(I1{}, I1{}, t + 1);
        t += 2;
    }
    if (t + 2 <= ksteps) {
        step(I0{}, I2{}, t);
        step(I1{}, I0{}, t + 1);
    }
    wait_vmcnt<0>();  // no copy may land in LDS once the epilogue reuses it

    // The MFMAs above are opaque to the compiler's hazard tracking: give the
    // last of them the wait states a matrix result needs before other
    // instructions read it (64, well above the 16x16x32 requirement).
    asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15\n\ts_nop 15" ::: "memory");
    ilv16_epilogue_t<T>(p, acc, smem, m0, n0, wm, wn, wave);
}

}  // namespace gsr
