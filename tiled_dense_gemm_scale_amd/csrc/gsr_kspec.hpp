// gsr_kspec.hpp -- the K-split small-tile kernel with the global -> LDS copies
// given to waves of their own (shapes with few output tiles: 256^3, 1024^3,
// the skinny class).
//
// Cycle counts taken inside the four-wave K-split kernel at 1024^3 show that
// issuing one K-step's buffer -> LDS copies holds a wave for ~700 clocks (a
// CU's vector-memory path accepts about 50 bytes of these copies per clock),
// that a wave cannot issue copies while its own MFMAs are queued, and so the
// copy issue and the MFMA issue of every step added up.  Here a workgroup has
// eight waves, two per SIMD: four copy waves that only issue copies and wait
// for them, and four MFMA waves that only read LDS and multiply, so one
// SIMD's MFMAs run while the other wave on it stalls on the memory path.
// Every wave passes the same barriers, one per K-step t:
//   copy wave:  wait until its copies of step t have landed; barrier t; send
//               the copies of step t + DEPTH into ring slot (t + DEPTH) %
//               STAGES, the slot of step t + DEPTH - STAGES (step t - 2 in
//               the compiled 4-slot, 2-deep form), whose reads every MFMA
//               wave finished before barrier t - 1.
//   MFMA wave:  barrier t (after its reads of step t - 1 have returned); read
//               step t; MFMAs of step t - 1.
// Tile, LDS operand layouts and the K split among the MFMA waves (wave w
// takes 16-k substeps w and w + 4 of each 128-deep step) are those of the
// four-wave K-split kernel, and the four partial tiles are summed in the same
// order, so the two kernels produce the same bits.  The sum runs on all eight
// waves: the MFMA waves write their partial tiles to LDS as row-major fp32
// rows (16-byte chunks XOR-swizzled by row, so neither the writes from the
// MFMA lane layout nor the row reads conflict), then each thread sums one
// row's eight consecutive outputs and stores them with one 16-byte store;
// eight lanes cover a 128-byte row of a 64-wide tile, so the stores write
// whole lines instead of 16-byte pieces of 32 rows.
//
// SPLIT (the entry points with a workspace): the K range of every tile is
// cut into p.ksplit runs of p.kchunk values, one workgroup each (workgroup
// id = part * tiles + tile), so shapes with few tiles still give every CU a
// workgroup.  A part runs the same K-steps over its own range; its sums then
// meet the other parts' in the workspace (KsSum::split_sum_store).
#pragma once

#include "gsr_ksplit.hpp"

namespace gsr {

template <int BM, int BN, int STAGES, int DEPTH, bool SPLIT>
__global__ void __launch_bounds__(512)
gemm_scale_relu_kspec_kernel(Problem p)
{
    using T = KsCfg<BM, BN, STAGES>;
    constexpr int BK = T::BK, NW = T::NW, CHA = T::CHA, CHN = T::CHN, TM = T::TM, TN = T::TN;
    static_assert(DEPTH >= 1 && DEPTH <= STAGES - 1, "steps in flight");

    __shared__ __attribute__((aligned(1024))) uint8_t smem[T::LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave8 = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool copier = wave8 >= NW;  // waves 4..7 copy, 0..3 multiply
    const int wave = wave8 & (NW - 1);

    // SPLIT: workgroup id = part * tiles + tile; part j covers K values
    // [j * kchunk, min(K, (j + 1) * kchunk))
    int tile = blockIdx.x, part = 0, kbeg = 0, kend = p.K;
    if constexpr (SPLIT) {
        const int tiles = p.tiles_m * p.tiles_n;
        part = blockIdx.x / tiles;
        tile = blockIdx.x - part * tiles;
        kbeg = part * p.kchunk;
        kend = min(p.K, kbeg + p.kchunk);
    }
    int tm, tn;
    tile_of(tile, SPLIT ? p.tiles_m * p.tiles_n : (int)gridDim.x, p, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int ksteps = (kend - kbeg + BK - 1) / BK;

    using Sum = KsSum<BM, BN, NW, 512>;  // the cross-wave sum runs on all eight waves
    static_assert(Sum::BYTES <= T::LDS_BYTES, "partial tiles fit in LDS");
    f32x4 bvs[Sum::NU][2];

    if (copier) {
        // ---- copy waves ----------------------------------------------------------
        const i32x4 ra = raw_rsrc(p.A, (uint32_t)p.M * (uint32_t)p.K * 2u);
        const i32x4 rb = raw_rsrc(p.B, (uint32_t)p.K * (uint32_t)p.N * 2u);
        const uint32_t lds0 = lds_address(smem);
        uint32_t a_off[T::A_PER];
        int a_k[T::A_PER];
        bool a_ok[T::A_PER];
#pragma unroll
        for (int i = 0; i < T::A_PER; ++i) {
            const int P = 64 * (wave + i * NW) + lane;
            const int r = P / CHA;
            const int c = (P % CHA) ^ (int)swz_a16((uint32_t)r);
            const int m = m0 + r;
            a_ok[i] = m < p.M;
            a_k[i] = 8 * c;
            a_off[i] = ((uint32_t)m * (uint32_t)p.K + (uint32_t)(kbeg + 8 * c)) * 2u;
        }
        uint32_t b_off[T::B_PER];
        int b_k[T::B_PER];
        bool b_ok[T::B_PER];
#pragma unroll
        for (int i = 0; i < T::B_PER; ++i) {
            const int P = 64 * (wave + i * NW) + lane;
            const int k = P / CHN;
            const int c = (P % CHN) ^ (int)swz_b<CHN>((uint32_t)k);
            const int n = n0 + 8 * c;
            b_ok[i] = n < p.N;
            b_k[i] = k;
            b_off[i] = ((uint32_t)(kbeg + k) * (uint32_t)p.N + (uint32_t)n) * 2u;
        }
        // k0: offset of the step from the part's first K value
        const int klen = kend - kbeg;
        auto issue = [&](int stage, int k0) {
            const uint32_t As = lds0 + stage * T::STAGE_BYTES;
            const uint32_t Bs = As + T::A_BYTES;
#pragma unroll
            for (int i = 0; i < T::A_PER; ++i) {
                const bool ok = a_ok[i] & (k0 + a_k[i] < klen);
                copy16_to_lds(ra, ok ? a_off[i] + (uint32_t)k0 * 2u : kOutOfRange, As + (wave + i * NW) * 1024);
            }
#pragma unroll
            for (int i = 0; i < T::B_PER; ++i) {
                const bool ok = b_ok[i] & (k0 + b_k[i] < klen);
                copy16_to_lds(rb, ok ? b_off[i] + (uint32_t)k0 * (uint32_t)p.N * 2u : kOutOfRange,
                              Bs + (wave + i * NW) * 1024);
            }
        };
#pragma unroll
        for (int s = 0; s < DEPTH; ++s)
            if (s < ksteps) issue(s, s * BK);
        for (int t = 0; t < ksteps; ++t) {
            // steps t+1 .. t+DEPTH-1 may still be in flight
            const int ahead = min(DEPTH - 1, ksteps - 1 - t);
            if (ahead == DEPTH - 1) wait_vmcnt<T::LOADS * (DEPTH - 1)>();
            else wait_vmcnt_dyn(T::LOADS * ahead);
            lds_barrier();
            if (t + DEPTH < ksteps) issue((t + DEPTH) % STAGES, (t + DEPTH) * BK);
        }
        Sum::load_bias(p, tid, n0, bvs);
        wait_vmcnt<0>();
        lds_barrier();  // the MFMA waves' partial tiles may now overwrite the buffers
    } else {
        // ---- MFMA waves ---------------------------------------------------------------
        const uint32_t frow = lane & 31, fhi = lane >> 5;
        uint32_t y_off[2][TM];  // A rows
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int b = 0; b < TM; ++b) {
                const uint32_t r = b * 32 + frow;
                const uint32_t c = 2u * (uint32_t)(wave + 4 * h) + fhi;
                y_off[h][b] = r * (BK * 2) + ((c ^ swz_a16(r)) << 4);
            }
        // transpose reads of B: 16-lane group G, i = l%16, e = i/4, q = i%4
        const uint32_t G = lane >> 4, li = lane & 15, e4 = li >> 2, q4 = li & 3;
        uint32_t x_off[2][2][TN];  // [substep half][read 0/1][n block]
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int rd = 0; rd < 2; ++rd)
#pragma unroll
                for (int a = 0; a < TN; ++a) {
                    const uint32_t k = 16u * (uint32_t)(wave + 4 * h) + 8u * (G >> 1) + 4u * rd + e4;
                    const uint32_t chunk = (uint32_t)(a * 32 + 16 * (G & 1)) / 8 + (q4 >> 1);
                    x_off[h][rd][a] = (uint32_t)T::A_BYTES + k * (BN * 2) + ((chunk ^ swz_b<CHN>(k)) << 4) + (q4 & 1) * 8;
                }

        f32x16 acc[TN][TM];
#pragma unroll
        for (int a = 0; a < TN; ++a)
#pragma unroll
            for (int b = 0; b < TM; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

        half8 xs0[2][TN], ys0[2][TM], xs1[2][TN], ys1[2][TM];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int a = 0; a < TN; ++a) xs0[h][a] = xs1[h][a] = (half8)(_Float16)0.0f;
#pragma unroll
            for (int b = 0; b < TM; ++b) ys0[h][b] = ys1[h][b] = (half8)(_Float16)0.0f;
        }
        auto read_step = [&](int stage, half8 (&xs)[2][TN], half8 (&ys)[2][TM]) {
            const uint8_t* base = smem + stage * T::STAGE_BYTES;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
                for (int b = 0; b < TM; ++b) ys[h][b] = __builtin_bit_cast(half8, *(const u32x4*)(base + y_off[h][b]));
#pragma unroll
                for (int a = 0; a < TN; ++a) {
                    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(base + x_off[h][0][a]));
                    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(base + x_off[h][1][a]));
                    xs[h][a] = __builtin_bit_cast(half8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                }
            }
        };
        auto mma_step = [&](const half8 (&xs)[2][TN], const half8 (&ys)[2][TM]) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int a = 0; a < TN; ++a)
#pragma unroll
                    for (int b = 0; b < TM; ++b)
                        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(xs[h][a], ys[h][b], acc[a][b], 0, 0, 0);
        };

        // step t is read into set t & 1 and multiplied one iteration later
        int t = 0;
        for (; t + 1 < ksteps; t += 2) {
            lds_barrier();
            read_step(t % STAGES, xs0, ys0);
            if (t > 0) mma_step(xs1, ys1);
            lds_barrier();
            read_step((t + 1) % STAGES, xs1, ys1);
            mma_step(xs0, ys0);
        }
        if (t < ksteps) {  // odd step count: one more even step
            lds_barrier();
            read_step(t % STAGES, xs0, ys0);
            if (t > 0) mma_step(xs1, ys1);
            mma_step(xs0, ys0);
        } else if (ksteps > 0) {
            mma_step(xs1, ys1);
        }

        Sum::load_bias(p, tid, n0, bvs);
        wait_vmcnt<0>();
        lds_barrier();  // every wave is done with the operand buffers
        Sum::write(smem, acc, wave, lane);
    }  // MFMA waves
    lds_barrier();  // partial tiles written

    // ---- every wave: sum, epilogue, one 16-byte store per unit --------------------
    if constexpr (SPLIT) {
        __shared__ int last;
        if (p.ksplit > 1) {
            Sum::split_sum_store(p, smem, &last, tid, m0, n0, bvs, tile, part);
            return;
        }
    }
    Sum::sum_store(p, smem, tid, m0, n0, bvs);
}

}  // namespace gsr
