// gsr_interleave_q.hpp -- the 128x128 tile of the explicitly interleaved
// 128-bit path of C = ReLU(alpha * A @ B), for shapes with a few hundred
// 128x128 tiles (e.g. 1024 x 4096 x 4096: 256 tiles of 128x128, 128 of
// 128x256, 64 of 256x256).
//
// The interleave design of gsr_interleave.hpp on a 128x128 tile: four waves, each
// owning 64x64 of the tile (2 x 2 accumulator blocks), two LDS stages (A and B
// 16 KiB each), A copied straight into LDS (4 copies per wave per step), every
// operand read 128 bits wide, both operands requested two K-steps ahead, one
// barrier per K-step.  B is one 8 (k) x 4 (n) block per thread, loaded as 8
// rows of 8 bytes and turned by byte permutes into 4 columns of 8 k, each
// written to LDS as one 16-byte store.  A 16-k substep has 4 MFMAs:
//   substep 0: the next substep's 4 operand reads, one per unit; from unit 1
//              the 16 permutes of the B(t+1) transpose;
//   substep 1: the next substep's reads, two B(t+2) row loads per unit;
//   substep 2: the next substep's reads, one transposed B(t+1) column write
//              per unit into the other stage;
//   substep 3: the wait + barrier after unit 0, then step t+1's 4 substep-0
//              reads and the 4 A(t+2) copies on units 1-3.
// LDS carries 96 KiB per K-step per CU against 512 MFMA cycles, so this tile
// is LDS-bound (the operand reads per MFMA double against 256x256); it pays
// where larger tiles leave CUs idle.  Ragged edges as in gsr_interleave.hpp.
#pragma once

#include "gsr_interleave.hpp"

namespace gsr {

struct IlvQCfg {
    static constexpr int BM = 128, BN = 128, BK = 64, WM = 2, WN = 2;
    static constexpr int NW = WM * WN, NT = kWave * NW;
    static constexpr int CH = BK / 8;
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    static constexpr int TM = WTM / 32, TN = WTN / 32;  // 2 x 2 accumulator blocks
    static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
    static constexpr int B_REGION = 2 * A_BYTES;
    static constexpr int LDS_BYTES = 2 * (A_BYTES + B_BYTES);
    static constexpr int A_PER = A_BYTES / 1024 / NW;  // 4 copies per wave per step
    static constexpr int B_LOADS = 8;                  // 8 rows of an 8x4 block per thread
    static constexpr int UNITS = TM * TN;              // MFMAs per substep
    static constexpr int READS = TM + TN;              // operand reads per substep
    static_assert((BK / 8) * (BN / 4) == NT, "one 8x4 B block per thread");
    static_assert(A_PER == 4 && UNITS == 4 && READS == 4, "the unit plan places 4 copies, 4 units, 4 reads");
};

// 8-byte global load into registers through a buffer descriptor (no compiler
// wait is attached: see wait_vmcnt_b8).
__device__ __forceinline__ u32x2 load8(i32x4 rsrc, uint32_t voff)
{
    u32x2 v;
    asm volatile("buffer_load_dwordx2 %0, %1, %2, 0 offen" : "=v"(v) : "v"(voff), "s"(rsrc) : "memory");
    return v;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt_b8(u32x2 (&r)[8])
{
    asm volatile("s_waitcnt vmcnt(%8)"
                 : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]), "+v"(r[4]), "+v"(r[5]), "+v"(r[6]), "+v"(r[7])
                 : "n"(N)
                 : "memory");
}

// permute q (0..15) of the 8x4 transpose: column c = q / 4 (= 2d + h), dword e = q % 4
__device__ __forceinline__ void transpose8x4_part(const u32x2 (&r)[8], u32x4 (&o)[4], int q)
{
    const int c = q >> 2, e = q & 3, d = c >> 1;
    o[c][e] = (c & 1) ? pack_hi(r[2 * e][d], r[2 * e + 1][d]) : pack_lo(r[2 * e][d], r[2 * e + 1][d]);
}

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_scale_relu_ilvq_kernel(Problem p)
{
    using T = IlvQCfg;
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
    // B block of this thread: rows kb*8..+7, columns nq*4..+3 of the tile
    // (N is a multiple of 8 on this path, so the 4 columns are in or out together)
    const uint32_t kb = (uint32_t)tid / (T::BN / 4), nq = (uint32_t)tid % (T::BN / 4);
    uint32_t b_voff[8];
    {
        const bool nok = (uint32_t)n0 + nq * 4u < N;
#pragma unroll
        for (int j = 0; j < 8; ++j) b_voff[j] = nok ? ((kb * 8u + (uint32_t)j) * N + nq * 4u) * 2u : kOutOfRange;
    }
    // transposed B writes: column nq*4+c of the tile, chunk kb
    uint32_t bw_addr[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const uint32_t r = nq * 4u + (uint32_t)c;
        bw_addr[c] = (uint32_t)T::B_REGION + r * (BK * 2) + ((kb ^ swz_a<CH>(r)) << 4);
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
    u32x2 breg[8];  // B block of a future step: 8 rows of 4 fp16
    u32x4 bcol[4];  // its transpose: 4 columns of 8 fp16

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
    // read i (0..3) of a substep's operands in the order its MFMAs need them:
    // x0, y0, y1 (units 0-1 use x0 with both y), then x1
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

        // substep 0: reads for substep 1; from unit 1 the transpose of B(t+1),
        // whose loads are in once at most the 4 copies of A(t+1) issued after
        // them are still in flight (16 permutes over units 1-3)
#pragma unroll
        for (int i = 0; i < T::UNITS; ++i) {
            mma(i, xf[0], yf[0]);
            read_next(S, 1, i, xf[1], yf[1]);
            if (i == 1) wait_vmcnt_b8<T::A_PER>(breg);
            if (i >= 1) {
#pragma unroll
                for (int q = (i - 1) * 16 / 3; q < i * 16 / 3; ++q) transpose8x4_part(breg, bcol, q);
            }
            sched_fence();
        }
        // substep 1: reads for substep 2, two B(t+2) row loads per unit
        {
            const i32x4 rb = b_rsrc(k2);
#pragma unroll
            for (int i = 0; i < T::UNITS; ++i) {
                mma(i, xf[1], yf[1]);
                read_next(S, 2, i, xf[0], yf[0]);
                breg[2 * i] = load8(rb, b_voff[2 * i]);
                breg[2 * i + 1] = load8(rb, b_voff[2 * i + 1]);
                sched_fence();
            }
        }
        // substep 2: reads for substep 3, one transposed B(t+1) column write per unit
#pragma unroll
        for (int i = 0; i < T::UNITS; ++i) {
            mma(i, xf[0], yf[0]);
            read_next(S, 3, i, xf[1], yf[1]);
            *(u32x4*)(smem + SN * T::B_BYTES + bw_addr[i]) = bcol[i];
            sched_fence();
        }
        // substep 3: publish step t+1 (A(t+1) landed: only the 8 B(t+2) loads
        // issued after its copies may be in flight; the B(t+1) writes and
        // every read of stage S are done), then step t+1's substep-0 reads and
        // the copies of A(t+2) into the freed stage S (reads 0-1 and copies
        // 0-1 on unit 1, then one of each on units 2 and 3)
        {
            const uint32_t kleft2 = (k2 < K) ? K - k2 : 0u;
            const i32x4 ra = a_rsrc(k2);
#pragma unroll
            for (int i = 0; i < T::UNITS; ++i) {
                mma(i, xf[1], yf[1]);
                if (i == 0) {
                    wait_vmcnt<T::B_LOADS>();
                    lds_barrier();
                } else {
                    const int lo = (i == 1) ? 0 : i, hi = i + 1;  // units 1, 2, 3 -> items {0,1}, {2}, {3}
#pragma unroll
                    for (int j = lo; j < hi; ++j) {
                        read_next(SN, 0, j, xf[0], yf[0]);
                        copy_a(S, j, kleft2, ra);
                    }
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
        for (int j = 0; j < 8; ++j) breg[j] = load8(rb, b_voff[j]);
        wait_vmcnt_b8<0>(breg);
#pragma unroll
        for (int q = 0; q < 16; ++q) transpose8x4_part(breg, bcol, q);
#pragma unroll
        for (int c = 0; c < 4; ++c) *(u32x4*)(smem + bw_addr[c]) = bcol[c];
        const i32x4 rb1 = b_rsrc((uint32_t)BK);
#pragma unroll
        for (int j = 0; j < 8; ++j) breg[j] = load8(rb1, b_voff[j]);
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
    wait_vmcnt_b8<0>(breg);

    ilv_epilogue<T>(p, acc, smem, m0, n0, wm, wn, wave, frow, fhi);
}

}  // namespace gsr
