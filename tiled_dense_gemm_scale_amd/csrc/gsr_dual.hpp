// gsr_dual.hpp -- the large-tile path of C = ReLU(alpha * A @ B) with both
// operands copied global -> LDS by the buffer unit and an explicit
// instruction interleave.
//
// Same tile, waves and accumulators as gsr_interleave.hpp (256x256x64, four
// waves of 128x128, 256 fp32 accumulators per lane), but B is not staged
// through registers: it is copied like A, straight into LDS as [BK][BN] rows,
// and each wave reads its B^T operands with the gfx950 transpose read
// (ds_read_b64_tr_b16, two reads per 16-k operand).  That drops the B loads
// into registers, their byte-permute transpose and the LDS writes from
// registers -- data movement that, on this part, costs clock: under a full
// MFMA load the engine clock is power-limited, so every byte staged through
// registers and LDS slows the MFMAs down.
//
// Per K-step t (four 16-k substeps of 16 MFMAs each), schedule units carry:
//   substeps 0-2: 12 operand reads for the next substep;
//   substep 3: three MFMAs, a wait for step t+1's copies and the barrier that
//              publishes them, then 12 operand reads of step t+1 (its substep
//              0) alongside all 16 copies of step t+2 into the stage the
//              barrier freed (two per unit on the first four units), so every
//              copy has a whole K-step to land.
// Operand read order in a substep: x0 (two halves), y0..y3, x1, x2, x3, so
// each lands well before the unit whose MFMA needs it.
#pragma once

#include "gsr_interleave.hpp"

namespace gsr {

struct DualCfg {
    using Base = IlvCfg;
    static constexpr int BM = Base::BM, BN = Base::BN, BK = Base::BK, WN = Base::WN;
    static constexpr int NW = Base::NW, NT = Base::NT, CH = Base::CH;
    static constexpr int CHN = BN / 8;                  // 32 chunks per B row (512 bytes)
    static constexpr int WTM = Base::WTM, WTN = Base::WTN, TM = Base::TM, TN = Base::TN;
    static constexpr int A_BYTES = Base::A_BYTES, B_BYTES = Base::B_BYTES;
    static constexpr int B_REGION = 2 * A_BYTES;        // A0 | A1 | B0 | B1
    static constexpr int LDS_BYTES = 2 * (A_BYTES + B_BYTES);
    static constexpr int A_PER = A_BYTES / 1024 / NW;   // 8 copies per wave per step
    static constexpr int B_PER = B_BYTES / 1024 / NW;   // 8
    static_assert(A_PER == 8 && B_PER == 8, "the unit plan places 8 + 8 copies");
    static_assert(LDS_BYTES == Base::LDS_BYTES, "same LDS footprint as the register-staged kernel");
    // ds_read offsets are 16-bit: stage and k offsets ride in the immediate
    static_assert(B_BYTES + (BK - 1) * BN * 2 < 65536, "B read offsets fit the immediate field");
};

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_scale_relu_dual_kernel(Problem p)
{
    using T = DualCfg;
    constexpr int BK = T::BK, CH = T::CH, CHN = T::CHN, TM = T::TM, TN = T::TN;

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
    const uint64_t a_base = (uint64_t)(uintptr_t)p.A + ((uint64_t)m0 * K) * 2u;
    const uint32_t a_recs = ((uint32_t)p.M * K - (uint32_t)m0 * K) * 2u;
    // B: base at (k0, n0), records up to the end of B: rows >= K are out.
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
    // Positioned at column k of A / row k of B; from k = K on they cover no
    // bytes at all, so every copy through them writes zeros.
    auto a_rsrc = [&](uint32_t k) { return (k < K) ? rsrc_of(a_base + (uint64_t)k * 2u, a_recs - k * 2u) : rsrc_of(a_base, 0u); };
    auto b_rsrc = [&](uint32_t k) {
        return (k < K) ? rsrc_of(b_base + (uint64_t)k * N * 2u, b_recs - k * N * 2u) : rsrc_of(b_base, 0u);
    };

    // ---- per-lane copy plan ------------------------------------------------
    // A copy i of this wave fills A chunk positions 64*(wave+4i) + lane: row
    // P / 8, physical chunk P % 8, logical chunk c = physical ^ swz_a(row).
    uint32_t a_voff[T::A_PER], a_kc[T::A_PER];
#pragma unroll
    for (int i = 0; i < T::A_PER; ++i) {
        const uint32_t P = 64u * (uint32_t)(wave + i * T::NW) + (uint32_t)lane;
        const uint32_t r = P / CH;
        const uint32_t c = (P % CH) ^ swz_a<CH>(r);
        a_voff[i] = (r * K + 8u * c) * 2u;
        a_kc[i] = 8u * c;
    }
    // B copy i fills B chunk positions 64*(wave+4i) + lane: row (k) P / 32,
    // physical chunk P % 32, logical chunk c = physical ^ swz_b(k); columns
    // past N read as zero (N is a multiple of 8, so a chunk is all in or out).
    uint32_t b_voff[T::B_PER];
#pragma unroll
    for (int i = 0; i < T::B_PER; ++i) {
        const uint32_t P = 64u * (uint32_t)(wave + i * T::NW) + (uint32_t)lane;
        const uint32_t k = P / CHN;
        const uint32_t c = (P % CHN) ^ swz_b<CHN>(k);
        b_voff[i] = ((uint32_t)n0 + 8u * c < N) ? (k * N + 8u * c) * 2u : kOutOfRange;
    }

    // ---- operand reads -----------------------------------------------------
    // A^T (second operand): lane l reads row (l % 32) of a 32-row block,
    // chunk 2*ks + l/32.
    const uint32_t frow = lane & 31, fhi = lane >> 5;
    uint32_t y_addr[4][TM];
#pragma unroll
    for (int b = 0; b < TM; ++b) {
        const uint32_t r = wm * T::WTM + b * 32 + frow;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) y_addr[ks][b] = r * (BK * 2) + (((2u * ks + fhi) ^ swz_a<CH>(r)) << 4);
    }
    // B^T (first operand) by transpose reads: 16-lane group G = l/16,
    // i = l%16, e = i/4, q = i%4; read rd (0, 1) of substep ks takes row
    // 16ks + 8(G/2) + 4rd + e, columns (block) + 16(G%2) + 4q..+3, and hands
    // lane i four k-consecutive values of column (block) + 16(G%2) + i.
    // Every such row is e (mod 4), so the swizzle of the row -- and with it
    // the lane's address -- differs between substeps, reads and stages only
    // by a constant.
    const uint32_t G = (uint32_t)lane >> 4, li = (uint32_t)lane & 15u, e4 = li >> 2, q4 = li & 3u;
    uint32_t x_base[TN];
#pragma unroll
    for (int a = 0; a < TN; ++a) {
        const uint32_t k = 8u * (G >> 1) + e4;  // row of read 0 in substep 0
        const uint32_t chunk = (uint32_t)(wn * T::WTN + a * 32 + 16 * (int)(G & 1u)) / 8u + (q4 >> 1);
        x_base[a] = (uint32_t)T::B_REGION + k * (T::BN * 2) + ((chunk ^ swz_b<CHN>(k)) << 4) + (q4 & 1u) * 8u;
    }

    f32x16 acc[TN][TM];
#pragma unroll
    for (int a = 0; a < TN; ++a)
#pragma unroll
        for (int b = 0; b < TM; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

    half8 xf[2][TN], yf[2][TM];  // two operand sets: substep parity
    v4i16 xlo[TN];               // first half of an x operand, waiting for its second

    // ---- building blocks ---------------------------------------------------
    auto copy_a = [&](int S, int i, uint32_t kleft, const i32x4& ra) {
        const uint32_t off = (a_kc[i] < kleft) ? a_voff[i] : kOutOfRange;
        copy16_to_lds(ra, off, lds0 + (uint32_t)(S * T::A_BYTES) + (uint32_t)(wave + i * T::NW) * 1024u);
    };
    auto copy_b = [&](int S, int i, const i32x4& rb) {
        copy16_to_lds(rb, b_voff[i], lds0 + (uint32_t)(T::B_REGION + S * T::B_BYTES) + (uint32_t)(wave + i * T::NW) * 1024u);
    };
    auto read_xh = [&](int S, int ks, int a, int rd) {
        const uint32_t off = (uint32_t)(S * T::B_BYTES + (16 * ks + 4 * rd) * T::BN * 2);
        return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(smem + x_base[a] + off));
    };
    // read j (0..11) of substep ks: x0 lo, x0 hi, y0, y1, y2, y3, x1 lo, x1 hi,
    // x2 lo, x2 hi, x3 lo, x3 hi
    auto read_op = [&](int S, int ks, int j, half8 (&xs)[TN], half8 (&ys)[TM]) {
        if (j >= 2 && j < 6) {
            const int b = j - 2;
            ys[b] = __builtin_bit_cast(half8, *(const u32x4*)(smem + S * T::A_BYTES + y_addr[ks][b]));
        } else {
            const int a = (j < 2) ? 0 : (j - 6) / 2 + 1;
            const int rd = (j < 2) ? j : (j - 6) % 2;
            const v4i16 h = read_xh(S, ks, a, rd);
            if (rd == 0) xlo[a] = h;
            else xs[a] = __builtin_bit_cast(half8, __builtin_shufflevector(xlo[a], h, 0, 1, 2, 3, 4, 5, 6, 7));
        }
    };
    auto mma = [&](int i, const half8 (&xs)[TN], const half8 (&ys)[TM]) {
        const int a = i / TM, b = i % TM;
        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(xs[a], ys[b], acc[a][b], 0, 0, 0);
    };

    // One K-step on stage S (its A and B are in LDS stage S, its substep-0
    // operands in xf[0]/yf[0]).  t is the step index.
    auto step = [&](auto stage_tag, int t) {
        constexpr int S = decltype(stage_tag)::value;
        constexpr int SN = S ^ 1;
        // substeps 0, 1 and 2: reads for the next substep
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            mma(i, xf[0], yf[0]);
            if (i < 12) read_op(S, 1, i, xf[1], yf[1]);
            sched_fence();
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            mma(i, xf[1], yf[1]);
            if (i < 12) read_op(S, 2, i, xf[0], yf[0]);
            sched_fence();
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            mma(i, xf[0], yf[0]);
            if (i < 12) read_op(S, 3, i, xf[1], yf[1]);
            sched_fence();
        }
        // substep 3: publish step t+1 (every copy of it is in: nothing was
        // issued after them), then its substep-0 reads and the sixteen copies of
        // step t+2 into the stage S just freed
        {
            const uint32_t k2 = (uint32_t)(t + 2) * BK;
            const uint32_t kleft2 = (k2 < K) ? K - k2 : 0u;
            const i32x4 ra2 = a_rsrc(k2);
            const i32x4 rb2 = b_rsrc(k2);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                mma(i, xf[1], yf[1]);
                if (i == 3) {
                    wait_vmcnt<0>();
                    lds_barrier();
                }
                if (i >= 4) {
                    read_op(SN, 0, i - 4, xf[0], yf[0]);
                    if (i < 12) copy_a(S, i - 4, kleft2, ra2);
                    if (i < 8) copy_b(S, i - 4, rb2);          // B 0..3 beside A 0..3
                    else if (i >= 12) copy_b(S, i - 8, rb2);   // B 4..7
                }
                sched_fence();
            }
        }
    };

    // ---- prologue: steps 0 and 1 in flight, step 0 published ----------------
    const int ksteps = (((int)K + BK - 1) / BK + 1) & ~1;  // even
    {
        const i32x4 ra0 = a_rsrc(0), rb0 = b_rsrc(0);
#pragma unroll
        for (int i = 0; i < T::A_PER; ++i) copy_a(0, i, K, ra0);
#pragma unroll
        for (int i = 0; i < T::B_PER; ++i) copy_b(0, i, rb0);
        const uint32_t k1 = (uint32_t)BK;
        const uint32_t kleft1 = (k1 < K) ? K - k1 : 0u;
        const i32x4 ra1 = a_rsrc(k1), rb1 = b_rsrc(k1);
#pragma unroll
        for (int i = 0; i < T::A_PER; ++i) copy_a(1, i, kleft1, ra1);
#pragma unroll
        for (int i = 0; i < T::B_PER; ++i) copy_b(1, i, rb1);
        wait_vmcnt<16>();  // step 0's sixteen copies are in
        lds_barrier();
#pragma unroll
        for (int j = 0; j < 12; ++j) read_op(0, 0, j, xf[0], yf[0]);
    }

    for (int t = 0; t < ksteps; t += 2) {
        step(std::integral_constant<int, 0>{}, t);
        step(std::integral_constant<int, 1>{}, t + 1);
    }
    wait_vmcnt<0>();  // no copy may land in LDS once the epilogue reuses it

    // ---- epilogue ------------------------------------------------------------
    ilv_epilogue(p, acc, smem, m0, n0, wm, wn, wave, frow, fhi);
}

}  // namespace gsr
