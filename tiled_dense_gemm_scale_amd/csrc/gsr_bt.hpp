// gsr_bt.hpp -- the large-tile 128-bit path of C = ReLU(alpha * A @ B).
//
// On gfx950 an LDS read instruction costs about the same LDS time whatever its
// width (a 64-bit read moves half the bytes of a 128-bit one in the same
// slot), so the cost of feeding the MFMAs is counted in LDS instructions.  This
// kernel keeps every MFMA operand read at 128 bits:
//  * A (K-contiguous) is copied global -> LDS by the buffer unit
//    (buffer_load_dwordx4 ... lds), rows of BK halves, 16-byte chunks
//    XOR-swizzled by row on the global side;
//  * B (N-contiguous) is loaded one step ahead into registers as 8x8 blocks,
//    transposed with byte permutes (VALU work that issues between MFMAs) and
//    written to LDS K-contiguous, rows of BK halves per column n, so its
//    operand reads are 128-bit too;
//  * four waves, each owning a 128x128 block of a 256x256 tile (the largest
//    accumulator the register file holds, 256 fp32 per lane): per 16-k
//    substep a wave issues 8 LDS reads for 16 MFMAs;
//  * operand fragments for substep s+1 are read while the MFMAs of substep s
//    run (two register sets).
// Ragged edges: out-of-range buffer loads return zero; out-of-range stores are
// dropped.
#pragma once

#include "gsr_pipeline.hpp"

namespace gsr {

template <int BM, int BN, int WM, int WN>
struct BtCfg {
    static constexpr int BK = 64;
    static constexpr int NW = WM * WN;
    static constexpr int NT = kWave * NW;
    static constexpr int CH = BK / 8;  // 16-byte chunks per LDS row (A and B)
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    static constexpr int TM = WTM / 32, TN = WTN / 32;
    static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
    static constexpr int LDS_BYTES = 2 * (A_BYTES + B_BYTES);
    static constexpr int A_PER = A_BYTES / 1024 / NW;          // DMA copies per wave per step
    static constexpr int B_BLOCKS = (BK / 8) * (BN / 8);       // 8x8 blocks per B tile
    static constexpr int B_PER = (B_BLOCKS + NT - 1) / NT;     // blocks per thread
    static constexpr int B_LOADS = 8 * B_PER;                  // vmem loads per thread per step

    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile");
    static_assert((A_BYTES / 1024) % NW == 0, "A copies split over waves");
    // every wave issues the same number of B loads, so one vmcnt fits all
    static_assert(B_BLOCKS % NT == 0, "B blocks split evenly over threads");
    static_assert(LDS_BYTES <= 163840, "LDS");
};

// The LDS footprint allows one workgroup per CU, i.e. one wave per SIMD: let the
// register allocator use the whole file for overlap instead of occupancy.
template <int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__(kWave * WM * WN) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_scale_relu_bt_kernel(Problem p)
{
    using T = BtCfg<BM, BN, WM, WN>;
    constexpr int BK = T::BK, NW = T::NW, NT = T::NT, CH = T::CH, TM = T::TM, TN = T::TN;

    __shared__ __attribute__((aligned(1024))) uint8_t smem[T::LDS_BYTES];
    // layout: A0 | A1 | B0 | B1
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;

    int tm, tn;
    tile_of(blockIdx.x, gridDim.x, p, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    const i32x4 ra = raw_rsrc(p.A, (uint32_t)p.M * (uint32_t)p.K * 2u);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.B, (uint32_t)p.K * (uint32_t)p.N * 2u);
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.C, (uint32_t)p.M * (uint32_t)p.N * 2u);
    const uint32_t lds0 = lds_address(smem);
    constexpr uint32_t B_REGION = 2 * T::A_BYTES;

    // ---- A copy plan (as in the pipelined kernel) ---------------------------
    uint32_t a_off[T::A_PER];
    int a_k[T::A_PER];
    bool a_ok[T::A_PER];
#pragma unroll
    for (int i = 0; i < T::A_PER; ++i) {
        const int j = wave + i * NW;
        const int P = 64 * j + lane;
        const int r = P / CH;
        const int c = (P % CH) ^ (int)swz_a<CH>(r);
        const int m = m0 + r;
        a_ok[i] = m < p.M;
        a_k[i] = 8 * c;
        a_off[i] = ((uint32_t)m * (uint32_t)p.K + (uint32_t)(8 * c)) * 2u;
    }
    auto issue_a = [&](int stage, int k0) {
        const uint32_t As = lds0 + stage * T::A_BYTES;
#pragma unroll
        for (int i = 0; i < T::A_PER; ++i) {
            const bool ok = a_ok[i] & (k0 + a_k[i] < p.K);
            const uint32_t off = ok ? a_off[i] + (uint32_t)k0 * 2u : kOutOfRange;
            copy16_to_lds(ra, off, As + (wave + i * NW) * 1024);
        }
    };

    // ---- B register plan: block (kb, nb) = rows kb*8.., columns nb*8.. -------
    constexpr int NB8 = BN / 8;
    u32x4 breg[T::B_PER][8];
    auto load_b = [&](int k0) {
#pragma unroll
        for (int i = 0; i < T::B_PER; ++i) {
            const int blk = tid + i * NT;
            if (T::B_BLOCKS % NT == 0 || blk < T::B_BLOCKS) {
                const int kb = blk / NB8, nb = blk % NB8;
                const int n = n0 + nb * 8;
                const bool nok = n < p.N;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int k = k0 + kb * 8 + j;
                    const uint32_t off = (nok & (k < p.K)) ? ((uint32_t)k * (uint32_t)p.N + (uint32_t)n) * 2u : kOutOfRange;
                    breg[i][j] = __builtin_amdgcn_raw_buffer_load_b128(rb, off, 0, 0);
                }
            }
        }
    };
    auto store_b = [&](int stage) {
        uint8_t* Bs = smem + B_REGION + stage * T::B_BYTES;
#pragma unroll
        for (int i = 0; i < T::B_PER; ++i) {
            const int blk = tid + i * NT;
            if (T::B_BLOCKS % NT == 0 || blk < T::B_BLOCKS) {
                const uint32_t kb = blk / NB8, nb = blk % NB8;
                u32x4 col[8];
                transpose8x8(breg[i], col);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const uint32_t r = nb * 8 + j;
                    *(u32x4*)(Bs + r * (BK * 2) + ((kb ^ swz_a<CH>(r)) << 4)) = col[j];
                }
            }
        }
    };

    // ---- fragment plan: 32x32x16 operands, lane l = row (l % 32) of its block,
    // chunk 2*ks + l/32 of the row ------------------------------------------------
    const uint32_t frow = lane & 31, fhi = lane >> 5;
    uint32_t x_row[TN], x_sw[TN], y_row[TM], y_sw[TM];
#pragma unroll
    for (int a = 0; a < TN; ++a) {
        const uint32_t r = wn * T::WTN + a * 32 + frow;
        x_row[a] = B_REGION + r * (BK * 2);
        x_sw[a] = swz_a<CH>(r);
    }
#pragma unroll
    for (int b = 0; b < TM; ++b) {
        const uint32_t r = wm * T::WTM + b * 32 + frow;
        y_row[b] = r * (BK * 2);
        y_sw[b] = swz_a<CH>(r);
    }
    auto read_frags = [&](int t, int ks, half8 (&xf)[TN], half8 (&yf)[TM]) {
        const uint8_t* As = smem + (t & 1) * T::A_BYTES;
        const uint8_t* Bs = smem + (t & 1) * T::B_BYTES;  // + B_REGION folded into x_row
        const uint32_t c = 2 * ks + fhi;
#pragma unroll
        for (int a = 0; a < TN; ++a)
            xf[a] = __builtin_bit_cast(half8, *(const u32x4*)(Bs + x_row[a] + ((c ^ x_sw[a]) << 4)));
#pragma unroll
        for (int b = 0; b < TM; ++b)
            yf[b] = __builtin_bit_cast(half8, *(const u32x4*)(As + y_row[b] + ((c ^ y_sw[b]) << 4)));
    };

    f32x16 acc[TN][TM];
#pragma unroll
    for (int a = 0; a < TN; ++a)
#pragma unroll
        for (int b = 0; b < TM; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

    const int ksteps = (p.K + BK - 1) / BK;

    // prologue: A(0) in flight, B(0) through registers into LDS, B(1) in flight
    issue_a(0, 0);
    load_b(0);
    store_b(0);
    if (ksteps > 1) load_b(BK);

    for (int t = 0; t < ksteps; ++t) {
        // A(t) is older than the B loads for step t+1 issued after it
        if (t + 1 < ksteps) wait_vmcnt<T::B_LOADS>();
        else wait_vmcnt<0>();
        lds_barrier();
        if (t + 1 < ksteps) issue_a((t + 1) & 1, (t + 1) * BK);

        half8 xf[2][TN], yf[2][TM];
        read_frags(t, 0, xf[0], yf[0]);
        __builtin_amdgcn_sched_group_barrier(0x100, TN + TM, 0);  // substep 0 reads lead
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            if (ks + 1 < BK / 16) read_frags(t, ks + 1, xf[(ks + 1) & 1], yf[(ks + 1) & 1]);
#pragma unroll
            for (int a = 0; a < TN; ++a)
#pragma unroll
                for (int b = 0; b < TM; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(xf[ks & 1][a], yf[ks & 1][b], acc[a][b], 0, 0, 0);
            // Issue order: the next substep's LDS reads spread between this
            // substep's MFMAs, so their latency hides behind MFMA execution.
            if (ks + 1 < BK / 16) {
#pragma unroll
                for (int i = 0; i < TN + TM; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
                }
                __builtin_amdgcn_sched_group_barrier(0x008, TN * TM - (TN + TM), 0);
            }
        }

        if (t + 1 < ksteps) store_b((t + 1) & 1);
        if (t + 2 < ksteps) load_b((t + 2) * BK);
    }

    // ---- epilogue ------------------------------------------------------------
    const float alpha = p.alpha;
    if (plain_epilogue(p)) {
#pragma unroll
        for (int a = 0; a < TN; ++a) {
#pragma unroll
            for (int b = 0; b < TM; ++b) {
                const int m = m0 + wm * T::WTM + b * 32 + (int)frow;
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int n = n0 + wn * T::WTN + a * 32 + 8 * g + 4 * (int)fhi;
                    half4 h;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float v = acc[a][b][4 * g + i] * alpha;
                        h[i] = (_Float16)(v > 0.0f ? v : 0.0f);
                    }
                    const uint32_t off = ((m < p.M) & (n < p.N)) ? ((uint32_t)m * (uint32_t)p.N + (uint32_t)n) * 2u : kOutOfRange;
                    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, h), rc, off, 0, 0);
                }
            }
        }
    } else {
        // bias of the lane's columns (all requested before the first use),
        // then act(alpha * acc + bias)
        const __amdgpu_buffer_rsrc_t rbias = bias_rsrc(p);
        f32x4 bvs[TN][4];
#pragma unroll
        for (int a = 0; a < TN; ++a)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                bvs[a][g] = p.bias ? bias4(rbias, n0 + wn * T::WTN + a * 32 + 8 * g + 4 * (int)fhi)
                                   : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        with_activation(p.act, [&](auto act_tag) {
            constexpr int ACT = decltype(act_tag)::value;
#pragma unroll
            for (int a = 0; a < TN; ++a) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int n = n0 + wn * T::WTN + a * 32 + 8 * g + 4 * (int)fhi;
                    const f32x4 bv = bvs[a][g];
#pragma unroll
                    for (int b = 0; b < TM; ++b) {
                        const int m = m0 + wm * T::WTM + b * 32 + (int)frow;
                        const f32x16 av = acc[a][b];
                        f32x4 sv;
#pragma unroll
                        for (int i = 0; i < 4; ++i) sv[i] = av[4 * g + i];
                        const half4 h = epilogue4<ACT>(sv, alpha, bv);
                        const uint32_t off = ((m < p.M) & (n < p.N)) ? ((uint32_t)m * (uint32_t)p.N + (uint32_t)n) * 2u : kOutOfRange;
                        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, h), rc, off, 0, 0);
                    }
                }
            }
        });
    }
}

}  // namespace gsr
