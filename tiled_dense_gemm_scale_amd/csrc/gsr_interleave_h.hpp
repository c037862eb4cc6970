// gsr_interleave_h.hpp -- the 128x256 tile of the explicitly interleaved
// 128-bit path of C = ReLU(alpha * A @ B), for mid-size shapes where 256x256
// tiles leave CUs idle (e.g. 2048 x 4096 x 4096: 256 tiles of 128x256, 128 of
// 256x256).
//
// The interleave design of gsr_interleave.hpp on a 128x256 tile: four
// waves, each owning 64x128 of the tile (2 x 4
// accumulator blocks, 128 fp32 accumulators per lane), two LDS stages (A
// 16 KiB + B 32 KiB each), A copied straight into LDS, B loaded into registers
// as one 8x8 block per thread, transposed with byte permutes and written
// K-contiguous, every operand read 128 bits wide, both operands requested two
// K-steps ahead, one barrier per K-step.  A 16-k substep has 8 MFMAs, so each
// schedule unit carries more companions:
//   substep 0: the next substep's 6 operand reads on units 0-5; from unit 2
//              the byte-permute transpose of B(t+1);
//   substep 1: the next substep's reads on units 0-5, one B(t+2) load per unit;
//   substep 2: the next substep's reads on units 0-5, one transposed B(t+1)
//              write per unit into the other stage;
//   substep 3: the wait + barrier after unit 1, then the 6 substep-0 reads of
//              step t+1 on units 2-7 and the 4 A(t+2) copies on units 2-5.
// The LDS carries 144 KiB per K-step per CU against 1024 MFMA cycles (a
// 256x256 tile: 192 KiB against 2048), so this tile is LDS-bound rather than
// MFMA-bound; it pays where it fills the chip and 256x256 does not.
// Ragged edges as in gsr_interleave.hpp.
#pragma once

#include "gsr_interleave.hpp"

namespace gsr {

struct IlvHCfg {
    static constexpr int BM = 128, BN = 256, BK = 64, WM = 2, WN = 2;
    static constexpr int NW = WM * WN, NT = kWave * NW;
    static constexpr int CH = BK / 8;
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    static constexpr int TM = WTM / 32, TN = WTN / 32;  // 2 x 4 accumulator blocks
    static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
    static constexpr int B_REGION = 2 * A_BYTES;
    static constexpr int LDS_BYTES = 2 * (A_BYTES + B_BYTES);
    static constexpr int A_PER = A_BYTES / 1024 / NW;  // 4 copies per wave per step
    static constexpr int B_LOADS = 8;                  // one 8x8 block per thread
    static constexpr int UNITS = TM * TN;              // MFMAs per substep
    static constexpr int READS = TM + TN;              // operand reads per substep
    static_assert((BK / 8) * (BN / 8) == NT, "one B block per thread");
    static_assert(A_PER == 4 && UNITS == 8 && READS == 6, "the unit plan places 4 copies, 8 units, 6 reads");
};

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_scale_relu_ilvh_kernel(Problem p)
{
    using T = IlvHCfg;
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

    // ---- descriptors that advance along K (as in the 256x256 kernel) -------
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

    // ---- per-lane copy plan --------------------------------------------------
    uint32_t a_voff[T::A_PER], a_kc[T::A_PER];
#pragma unroll
    for (int i = 0; i < T::A_PER; ++i) {
        const uint32_t P = 64u * (uint32_t)(wave + i * T::NW) + (uint32_t)lane;
        const uint32_t r = P / CH;
        const uint32_t c = (P % CH) ^ swz_a<CH>(r);
        a_voff[i] = (r * K + 8u * c) * 2u;
        a_kc[i] = 8u * c;
    }
    const uint32_t kb = (uint32_t)tid / (T::BN / 8), nb = (uint32_t)tid % (T::BN / 8);
    uint32_t b_voff[8];
    {
        const bool nok = (uint32_t)n0 + nb * 8u < N;
#pragma unroll
        for (int j = 0; j < 8; ++j) b_voff[j] = nok ? ((kb * 8u + (uint32_t)j) * N + nb * 8u) * 2u : kOutOfRange;
    }
    uint32_t bw_addr[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t r = nb * 8u + (uint32_t)j;
        bw_addr[j] = (uint32_t)T::B_REGION + r * (BK * 2) + ((kb ^ swz_a<CH>(r)) << 4);
    }
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

    half8 xf[2][TN], yf[2][TM];
    u32x4 breg[8];
    u32x4 bcol[8];

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
    // read i (0..5) of a substep's operands in the order its MFMAs need them:
    // x0, y0, y1 (units 0-1 use x0 with both y), then x1..x3
    auto read_next = [&](int S, int ks, int i, half8 (&xs)[TN], half8 (&ys)[TM]) {
        if (i == 0) read_x(S, ks, 0, xs[0]);
        else if (i <= TM) read_y(S, ks, i - 1, ys[i - 1]);
        else read_x(S, ks, i - TM, xs[i - TM]);
    };
    auto mma = [&](int i, const half8 (&xs)[TN], const half8 (&ys)[TM]) {
        const int a = i / TM, b = i % TM;
        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(xs[a], ys[b], acc[a][b], 0, 0, 0);
    };

    // One K-step on stage S (its A and B in LDS stage S, its substep-0
    // operands in xf[0]/yf[0]); t is the step index.
    auto step = [&](auto stage_tag, int t) {
        constexpr int S = decltype(stage_tag)::value;
        constexpr int SN = S ^ 1;
        const uint32_t k2 = (uint32_t)(t + 2) * BK;

        // substep 0: reads for substep 1; from unit 2 the transpose of B(t+1),
        // whose loads are in once at most the 4 copies of A(t+1) issued after
        // them are still in flight (16 (e, d) permute pairs over units 2-7)
#pragma unroll
        for (int i = 0; i < T::UNITS; ++i) {
            mma(i, xf[0], yf[0]);
            if (i < T::READS) read_next(S, 1, i, xf[1], yf[1]);
            if (i == 2) wait_vmcnt_b<T::A_PER>(breg);
            if (i >= 2) {
#pragma unroll
                for (int q = (i - 2) * 16 / 6; q < (i - 1) * 16 / 6; ++q) {
                    const int e = q >> 2, d = q & 3;
                    bcol[2 * d][e] = pack_lo(breg[2 * e][d], breg[2 * e + 1][d]);
                    bcol[2 * d + 1][e] = pack_hi(breg[2 * e][d], breg[2 * e + 1][d]);
                }
            }
            sched_fence();
        }
        // substep 1: reads for substep 2, one B(t+2) load per unit
        {
            const i32x4 rb = b_rsrc(k2);
#pragma unroll
            for (int i = 0; i < T::UNITS; ++i) {
                mma(i, xf[1], yf[1]);
                if (i < T::READS) read_next(S, 2, i, xf[0], yf[0]);
                breg[i] = load16(rb, b_voff[i]);
                sched_fence();
            }
        }
        // substep 2: reads for substep 3, one transposed B(t+1) write per unit
#pragma unroll
        for (int i = 0; i < T::UNITS; ++i) {
            mma(i, xf[0], yf[0]);
            if (i < T::READS) read_next(S, 3, i, xf[1], yf[1]);
            *(u32x4*)(smem + SN * T::B_BYTES + bw_addr[i]) = bcol[i];
            sched_fence();
        }
        // substep 3: publish step t+1 (A(t+1) landed: only the 8 B(t+2) loads
        // issued after its copies may be in flight; the B(t+1) writes and
        // every read of stage S are done), then step t+1's substep-0 reads and
        // the copies of A(t+2) into the freed stage S
        {
            const uint32_t kleft2 = (k2 < K) ? K - k2 : 0u;
            const i32x4 ra = a_rsrc(k2);
#pragma unroll
            for (int i = 0; i < T::UNITS; ++i) {
                mma(i, xf[1], yf[1]);
                if (i == 1) {
                    wait_vmcnt<T::B_LOADS>();
                    lds_barrier();
                }
                if (i >= 2) {
                    read_next(SN, 0, i - 2, xf[0], yf[0]);
                    if (i - 2 < T::A_PER) copy_a(S, i - 2, kleft2, ra);
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
        for (int i = 0; i < T::READS; ++i) read_next(0, 0, i, xf[0], yf[0]);
    }

    for (int t = 0; t < ksteps; t += 2) {
        step(std::integral_constant<int, 0>{}, t);
        step(std::integral_constant<int, 1>{}, t + 1);
    }
    // drain every load before the epilogue (see the 256x256 kernel)
    wait_vmcnt_b<0>(breg);

    ilv_epilogue<T>(p, acc, smem, m0, n0, wm, wn, wave, frow, fhi);
}

}  // namespace gsr
