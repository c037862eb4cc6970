// gsr_interleave16.hpp -- the 256x256 explicitly interleaved kernel on the
// 16x16x32 fp16 MFMA with B transposed through registers (configuration 25),
// and the 16x16x32 fragment MFMA and epilogue that the kernel of
// gsr_interleave16d.hpp (configuration 28, B copied to LDS and read with
// transpose reads) shares.  The selector runs configuration 28, which gives
// this kernel's bits faster; this one is kept as its register-transpose twin.
//
// The 256x256 tile of the interleave design (gsr_interleave.hpp): four waves
// of 128x128, two LDS stages, A copied straight into LDS, B loaded into
// registers one 8x8 block per thread, transposed with byte permutes and
// written K-contiguous, one barrier per K-step.  Why 16x16x32 MFMAs: with
// random fp16 operands the part runs power-limited, and a chip-wide stream of
// v_mfma_f32_16x16x32_f16 holds a markedly higher engine clock than the same
// FLOP issued as v_mfma_f32_32x32x16_f16 (both at their full issue rate:
// ~1.7-1.8 vs ~1.4-1.5 GHz), so where enough CUs run for that limit to bind
// it finishes the same work sooner even though its 16-cycle MFMAs leave half
// the issue shadow for the other instructions of a K-step.
//
// Each wave owns 128x128 of the tile as 8 x 8 accumulator blocks of 16x16
// (four fp32 per lane each, all 256 in AGPRs).  A K-step (BK = 64) is two
// 32-deep substeps of 64 MFMAs; MFMA slot i of a substep multiplies the
// B^T fragment X[i / 8] with the A^T fragment Y[i % 8].  A fragment is one
// 128-bit LDS read: lane l takes row (l % 16) of a 16-row block and one
// 16-byte chunk of the substep's four (A and B^T are both K-contiguous in
// LDS, 16-byte chunks XOR-swizzled by row).
//
// Operand registers: one set of X[0..6] (an X fragment is refilled for the
// next substep as soon as its eight MFMAs have issued), two of X[7] and two Y
// sets (all eight Y fragments are used across the whole substep).  Each
// substep reads the next substep's operands: X[a] at slot 8a + 8, X[7] at slot
// 44 (substep 0) or 60 (substep 1), Y[b] every fourth slot from slot 2
// (substep 0) or 10 (substep 1, after the barrier).  The barrier waits for
// this wave's LDS operations: the last read before it is 14 slots old, the
// last B^T write 8.  Spreading the companions evenly over the slots matters
// as much as what they are (one MFMA every 16 cycles cannot wait on a burst).
//
// Companions of step t on stage S (SN = S ^ 1):
//   substep 0, slots 16-31: wait for B(t+1), transpose it in registers;
//   substep 0, slots 34-62 (every 4th): write B(t+1)^T into stage SN;
//   substep 0, slots 35-63 (every 4th): load B(t+2) into registers;
//   substep 1, slot 6:   wait for the A(t+1) copies, barrier (publishes
//                        stage SN, frees stage S);
//   substep 1, slots 7-35 (every 4th): copy A(t+2) into stage S;
//   substep 1 reads (from slot 8 on) come from stage SN (step t+1).
#pragma once

#include <type_traits>

#include "gsr_interleave.hpp"

namespace gsr {

struct Ilv16Cfg : IlvCfg {
    static constexpr int FM = WTM / 16, FN = WTN / 16;  // 8 x 8 blocks of 16x16
};

// acc += x^T-block * y-block on the 16x16x32 fp16 MFMA, with the accumulator
// pinned to AGPRs and updated in place.  (Through the compiler builtin the
// register allocator spreads 64 four-register accumulators over AGPRs and
// VGPRs and copies them around every MFMA.)  Operands only come from LDS
// reads, whose completion the compiler still waits for, and accumulators are
// never written by any other instruction inside the loop.
__device__ __forceinline__ void mfma16_inplace(f32x4& acc, const half8& x, const half8& y)
{
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(x), "v"(y));
}

// Epilogue of the 16x16 layout, for a WTM x WTN wave sub-tile (WTN = 128 or
// 64): lane l holds, for accumulator block (a, b), rows m = 16b + l % 16 and
// columns n = 16a + 4(l / 16) + 0..3 of the sub-tile.  Scale, ReLU (or the
// variant) and round in registers, stage each wave's fp16 sub-tile in its own
// LDS rows (16-byte chunk c of row r at physical chunk c ^ (r mod WTN / 8)),
// then store whole row segments of 2 WTN bytes.  Called once every wave's
// copies have been drained.
template <class T>
__device__ __forceinline__ void ilv16_epilogue_t(const Problem& p, const f32x4 (&acc)[T::FN][T::FM], uint8_t* smem,
                                                 int m0, int n0, int wm, int wn, int wave)
{
    constexpr int FM = T::FM, FN = T::FN;
    const uint32_t lane = (uint32_t)(threadIdx.x & 63);
    const uint32_t lrow = lane & 15u, lq = lane >> 4;
    const uint32_t N = (uint32_t)p.N;
    constexpr uint32_t CPR = T::WTN / 8, RB = T::WTN * 2;  // chunks and bytes per staging row
    static_assert((T::WTN == 128 || T::WTN == 64) && T::NW * T::WTM * T::WTN * 2 <= T::LDS_BYTES,
                  "staging rows of 8 or 16 chunks fit");
    const bool plain = plain_epilogue(p);
    f32x4 bvs[FN];
    {
        const __amdgpu_buffer_rsrc_t rbias = bias_rsrc(p);
        const bool load = !plain && p.bias != nullptr;
#pragma unroll
        for (int a = 0; a < FN; ++a)
            bvs[a] = load ? bias4(rbias, n0 + wn * T::WTN + a * 16 + 4 * (int)lq) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    lds_barrier();  // every wave is past its last operand read
    const float alpha = p.alpha;
    uint8_t* const ep = smem + wave * (T::WTM * T::WTN * 2);
    auto stage4 = [&](int a, int b, half4 h) {
        const uint32_t r = (uint32_t)b * 16u + lrow;
        const uint32_t c = ((uint32_t)(2 * a) + (lq >> 1)) ^ (r & (CPR - 1u));
        *(u32x2*)(ep + r * RB + c * 16u + (lq & 1u) * 8u) = __builtin_bit_cast(u32x2, h);
    };
    if (plain) {
#pragma unroll
        for (int a = 0; a < FN; ++a)
#pragma unroll
            for (int b = 0; b < FM; ++b) {
                half4 h;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float v = acc[a][b][i] * alpha;
                    h[i] = (_Float16)(v > 0.0f ? v : 0.0f);
                }
                stage4(a, b, h);
            }
    } else {
        with_activation(p.act, [&](auto act_tag) {
            constexpr int ACT = decltype(act_tag)::value;
#pragma unroll
            for (int a = 0; a < FN; ++a)
#pragma unroll
                for (int b = 0; b < FM; ++b) stage4(a, b, epilogue4<ACT>(acc[a][b], alpha, bvs[a]));
        });
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.C, (uint32_t)p.M * N * 2u);
    constexpr uint32_t RPI = 64u / CPR;  // rows per store instruction
    const uint32_t sc = lane & (CPR - 1u);
    const int n = n0 + wn * T::WTN + 8 * (int)sc;
    // C is written once and never read back here: the stores carry the
    // non-temporal hint (cache policy bit 1, `nt`).  Interleaved timings on one
    // MI355X, same bits: 0.2-2 % faster at 4096^3, 3072^3, 16384^3, the
    // LLM shape and 2048 x 4096 x 4096, in either timing order.
    constexpr int kStoreNonTemporal = 2;
    // C at a 16-byte aligned address takes one 16-byte store per row segment;
    // a less aligned C, the stores its alignment allows (p.unit_c)
    with_store_unit(p.unit_c, [&](auto unit_tag) {
        constexpr int U = decltype(unit_tag)::value;
#pragma unroll
        for (int j = 0; j < (int)(T::WTM / RPI); ++j) {
            const uint32_t r = RPI * (uint32_t)j + lane / CPR;
            const u32x4 v = *(const u32x4*)(ep + r * RB + ((sc ^ (r & (CPR - 1u))) << 4));
            const int m = m0 + wm * T::WTM + (int)r;
            const uint32_t off = ((m < p.M) & (n < p.N)) ? ((uint32_t)m * N + (uint32_t)n) * 2u : kOutOfRange;
            store16_unit<U, kStoreNonTemporal>(v, rc, off);
        }
    });
}

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_scale_relu_ilv16_kernel(Problem p)
{
    using T = Ilv16Cfg;
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

    // ---- descriptors that advance along K -----------------------------------
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
    // Kept in a few base registers: a 256-thread tile has no room for
    // eight-entry offset tables beside the operand sets.
    // A copy i of this wave fills LDS chunk positions 64*(wave+4i) + lane: row
    // r = 8*wave + 32i + lane/8, physical chunk lane % 8, logical chunk
    // c = (lane % 8) ^ swz(r) = c0 ^ 4*(i & 1) with c0 below.
    const uint32_t c0 = ((uint32_t)lane & 7u) ^ ((uint32_t)lane >> 3) ^ (uint32_t)wave;
    const uint32_t arow = (8u * (uint32_t)wave + ((uint32_t)lane >> 3)) * K * 2u;
    // byte offsets of copies 0 and 1 (32 rows apart) and their first k; copy
    // i is copy i % 2 moved down 64 * (i / 2) rows
    uint32_t av0 = arow + 16u * c0, av1 = arow + 32u * K * 2u + 16u * (c0 ^ 4u);
    uint32_t kc0 = 8u * c0, kc1 = 8u * (c0 ^ 4u);
    const uint32_t a_istride = 64u * K * 2u;
    // B block of this thread: rows kb*8..+7, columns nb*8..+7 of the tile; row j
    // of the block is N elements after row j - 1 (no wrap: every offset of B
    // stays below 2^31 bytes, so kOutOfRange + j*N*2 stays out of range).
    const uint32_t kb = (uint32_t)tid / (T::BN / 8), nb = (uint32_t)tid % (T::BN / 8);
    uint32_t b_off0 = ((uint32_t)n0 + nb * 8u < N) ? ((kb * 8u) * N + nb * 8u) * 2u : kOutOfRange;
    // transposed B write j: row nb*8 + j of the B^T tile, chunk kb ^ swz(row)
    // = (kb ^ nb ^ j) & 7, i.e. bwq ^ (j << 4) plus j*128 bytes.
    uint32_t bwq = (uint32_t)T::B_REGION + nb * 8u * (BK * 2) + (((kb ^ nb) & 7u) << 4);
    // Fragment addresses (stage 0, substep 0) of the B^T blocks a = 0..3.
    // Block a + 4 is 64 rows (8 KiB) further with the same swizzle; substep 1
    // flips chunk bit 2 (byte offset ^ 64); the A block b of this wave has the
    // same swizzle as B^T block b (the rows differ by a multiple of 128), so
    // its address is the B^T one minus a wave-uniform distance.
    // Lane group g = l / 16 takes k-group chunk (g & 1) * 2 + g / 2 of its
    // substep (the same permutation for both operands, so every product pairs
    // the same k): the LDS serves lanes l and l + 32 of a 128-bit read
    // together, and their rows must then differ in chunk bit 0, which keeps
    // every read free of bank conflicts (with chunks g in order, lanes 0-7 and
    // 32-39 collide two-way).
    const uint32_t lrow = (uint32_t)lane & 15u, lq = (uint32_t)lane >> 4;
    const uint32_t lch = ((lq & 1u) << 1) | (lq >> 1);
    uint32_t xb[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const uint32_t rx = (uint32_t)wn * T::WTN + (uint32_t)a * 16u + lrow;
        xb[a] = (uint32_t)T::B_REGION + rx * (BK * 2) + ((lch ^ swz_a<CH>(rx)) << 4);
    }
    const uint32_t ydelta = (uint32_t)T::B_REGION + (uint32_t)((wn - wm) * T::WTN * (BK * 2));

    f32x4 acc[FN][FM];
#pragma unroll
    for (int a = 0; a < FN; ++a)
#pragma unroll
        for (int b = 0; b < FM; ++b) acc[a][b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    half8 X[FN - 1];  // B^T fragments 0..6, refilled one by one
    half8 X7[2];      // B^T fragment 7, one per substep parity
    half8 Y[2][FM];   // A^T fragments, one set per substep parity
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
        const uint32_t off = (xb[b & 3] ^ (ks ? 64u : 0u)) - ydelta;
        dst = __builtin_bit_cast(half8, *(const u32x4*)(smem + S * T::A_BYTES + (b >> 2) * (64 * BK * 2) + off));
    };
    // The reads of slot i of a substep, all for the next substep (stage SR,
    // substep kr): X[a] (a < 7) at slot 8a + 8, as soon as its last MFMA here
    // has issued; X[7] (into the other X7 register) at slot x7; Y[b] at slot
    // y0 + 4b, at least 30 slots before its first use.
    auto reads = [&](int i, int SR, int kr, half8 (&ynext)[FM], int y0, int x7) {
        if ((i & 7) == 0 && i >= 8 && i <= 8 * (FN - 1)) read_x(SR, kr, (i >> 3) - 1);
        if (i == x7) read_x(SR, kr, FN - 1);
        if (i >= y0 && i < y0 + 4 * FM && ((i - y0) & 3) == 0) read_y(SR, kr, (i - y0) >> 2, ynext[(i - y0) >> 2]);
    };
    auto mma = [&](int i, int ks, const half8 (&ys)[FM]) {
        const int a = i >> 3;
        mfma16_inplace(acc[a][i & 7], a == FN - 1 ? X7[ks] : X[a], ys[i & 7]);
    };

    auto step = [&](auto stage_tag, int t) {
        constexpr int S = decltype(stage_tag)::value;
        constexpr int SN = S ^ 1;
        const uint32_t k2 = (uint32_t)(t + 2) * BK;
        // Opaque to the optimiser from here on: the per-copy and per-write
        // offsets derived from these are then formed where they are used
        // instead of being hoisted out of the loop into live registers.
        asm volatile("" : "+v"(av0), "+v"(av1), "+v"(kc0), "+v"(kc1), "+v"(b_off0), "+v"(bwq), "+v"(xb[0]), "+v"(xb[1]),
                     "+v"(xb[2]), "+v"(xb[3]));
        // substep 0 (Y[0]); reads for substep 1 of this step
        {
            const i32x4 rb = b_rsrc(k2);
#pragma unroll
            for (int i = 0; i < 64; ++i) {
                mma(i, 0, Y[0]);
                reads(i, S, 1, Y[1], 2, 44);
                if (i == 16) wait_vmcnt_b<T::A_PER>(breg);  // B(t+1) is in; A(t+1) copies may not be
                if (i >= 16 && i < 32) {
                    // one of the 16 byte-permute pairs (two permutes) per slot
                    const int e = (i - 16) >> 2, d = (i - 16) & 3;
                    bcol[2 * d][e] = pack_lo(breg[2 * e][d], breg[2 * e + 1][d]);
                    bcol[2 * d + 1][e] = pack_hi(breg[2 * e][d], breg[2 * e + 1][d]);
                }
                if (i >= 34 && (i & 3) == 2) write_bt(SN, (i - 34) >> 2);
                if (i >= 35 && (i & 3) == 3) breg[(i - 35) >> 2] = load16(rb, b_voff((i - 35) >> 2));
                sched_fence();
            }
        }
        // substep 1 (Y[1]); after the barrier, reads for substep 0 of step t+1
        {
            const uint32_t kleft2 = (k2 < K) ? K - k2 : 0u;
            const i32x4 ra = a_rsrc(k2);
#pragma unroll
            for (int i = 0; i < 64; ++i) {
                mma(i, 1, Y[1]);
                if (i == 6) {
                    wait_vmcnt<T::B_LOADS>();  // A(t+1) copies are in; B(t+2) loads may not be
                    lds_barrier();
                }
                reads(i, SN, 0, Y[0], 10, 60);
                if (i >= 7 && i < 39 && (i & 3) == 3) copy_a(S, (i - 7) >> 2, kleft2, ra);
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

    // The MFMAs above are opaque to the compiler's hazard tracking: give the
    // last of them the wait states a matrix result needs before other
    // instructions read it (64, well above the 16x16x32 requirement).
    asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15\n\ts_nop 15" ::: "memory");
    ilv16_epilogue_t<T>(p, acc, smem, m0, n0, wm, wn, wave);
}

}  // namespace gsr
