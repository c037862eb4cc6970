// gsr_pipeline.hpp -- the 128-bit path: C = ReLU(alpha * A @ B) with A and B
// copied global -> LDS by the buffer unit itself (no register staging), a ring
// of STAGES LDS buffers kept STAGES-1 K-steps ahead of the MFMAs, and B
// transposed by the gfx950 LDS transpose read.
//
// Design notes (CDNA4 / gfx950):
//  * buffer_load_dwordx4 ... lds writes lane L's 16 bytes to LDS at
//    base + 16*L.  Every wave-wide copy therefore fills 1 KiB of LDS
//    contiguously; the bank-conflict swizzle is applied on the global side by
//    choosing which 16-byte chunk each lane fetches.  Out-of-range chunks
//    (ragged M, N or K) read as zero, so the tile maths never sees garbage.
//  * A is K-contiguous and lands as [BM][BK] rows; a lane's MFMA operand is
//    one 128-bit LDS read.
//  * B is N-contiguous and lands as [BK][BN] rows.  ds_read_b64_tr_b16 gives,
//    within each 16-lane group, output lane i element e = source lane
//    (4e + i/4) element (i % 4): when source lane 4e+q points at row k0+e,
//    columns n0+4q..n0+4q+3, lane i receives B[k0..k0+3][n0+i], i.e. four
//    K-consecutive values of one column.  Two such reads form the eight
//    values of a 32x32x16 MFMA operand.
//  * The MFMA takes B^T as its first operand and A^T as its second, so an
//    accumulator block holds four consecutive n per lane and register group.
//  * Synchronisation per K-step: wait for this wave's copies of the step,
//    one barrier (everyone's copies landed; everyone finished reading the
//    buffer about to be refilled), issue the copies STAGES-1 steps ahead,
//    then the MFMAs of the step.
#pragma once

#include "gsr_kernels.hpp"

namespace gsr {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

typedef int i32x4 __attribute__((ext_vector_type(4)));

// The copies, the waits on them and the barrier are issued as inline asm with
// a "memory" clobber: the compiler then neither hoists LDS reads across them
// nor adds its own conservative vmcnt(0) waits (it would otherwise wait for
// every outstanding copy before each LDS read, which serialises the ring).
// Vector-memory operations retire in order, so waits the compiler emits for
// its own loads can only become stricter, never wrong.

// Buffer resource for a raw byte range (gfx9-family descriptor: base address,
// stride 0, num_records = bytes, data-format word).
__device__ __forceinline__ i32x4 raw_rsrc(const void* p, uint32_t bytes)
{
    const uint64_t a = (uint64_t)(uintptr_t)p;
    i32x4 r;
    r[0] = (int)(uint32_t)a;
    r[1] = (int)((uint32_t)(a >> 32) & 0xffffu);
    r[2] = (int)bytes;
    r[3] = 0x00020000;
    return r;
}

// Copy 16 bytes per lane from the buffer at byte offset voff (out of range
// reads zero) into LDS at lds_addr + 16 * lane.
__device__ __forceinline__ void copy16_to_lds(i32x4 rsrc, uint32_t voff, uint32_t lds_addr)
{
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :: "v"(voff), "s"(rsrc), "s"(lds_addr) : "memory", "m0");
}

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

__device__ __forceinline__ void wait_vmcnt_dyn(int n)
{
    // n is uniform and small; fall back to stricter waits past 8
    if (n <= 0) wait_vmcnt<0>();
    else if (n == 1) wait_vmcnt<1>();
    else if (n == 2) wait_vmcnt<2>();
    else if (n == 3) wait_vmcnt<3>();
    else if (n < 6) wait_vmcnt<4>();
    else if (n < 8) wait_vmcnt<6>();
    else if (n < 12) wait_vmcnt<8>();
    else if (n < 16) wait_vmcnt<12>();
    else if (n < 24) wait_vmcnt<16>();
    else if (n < 32) wait_vmcnt<24>();
    else wait_vmcnt<32>();
}

// Barrier after this wave's LDS reads have returned (so no wave refills a
// buffer another wave is still reading).
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ uint32_t lds_address(const void* p)
{
    return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const uint8_t*)p);
}

// A tile rows of BK halves: 16-byte chunk c of row r sits at chunk c ^ swz_a(r).
template <int CH>
__device__ __forceinline__ uint32_t swz_a(uint32_t r)
{
    if constexpr (CH == 8) return (r ^ (r >> 3)) & 7u;
    else return ((r >> 1) ^ (r >> 2)) & 3u;  // CH == 4
}

// B tile rows (one k each) of BN halves: chunk c of row k sits at c ^ swz_b(k).
// A transpose read hands each 16-lane group rows k..k+3 of a 16-k substep
// (k = 8g' + 4r, g' = lane group / 2) and two 16-byte chunks per row, the
// group next to it the next two chunks of the same rows.
//  * 128-byte rows (BN = 64): the LDS serves 64 banks of 4 bytes per cycle,
//    so even rows fall on one half of the banks and odd rows on the other, and
//    rows k and k + 8 are read by the same instruction.  Masks (2(k mod 4)) ^
//    (2 if k mod 16 >= 8) give the rows served together disjoint chunks
//    whether the cycle takes lanes 0-31 (rows k..k+3, four chunks each) or
//    lanes 0-15 with 32-47 (rows k..k+3 and k+8..k+11, two chunks each), and
//    also when 16 lanes are served per cycle.  The masks 0, 6, 2, 4 by
//    k mod 4 used before repeat every four rows, which left rows k and k + 2
//    (and k and k + 8) on the same banks: two extra cycles per read
//    (rocprofv3 SQ_LDS_BANK_CONFLICT, one cycle per LDS instruction on the
//    64x64 K-split kernel at 1024^3).
//  * other widths: four consecutive rows get XOR masks whose bits 1-2 and
//    bits 2-3 are both distinct, which spreads a read's 4 rows x 2-4 chunks
//    over the banks.
template <int CHN>
__device__ __forceinline__ uint32_t swz_b(uint32_t k)
{
    if constexpr (CHN == 8) return ((k & 3u) << 1) ^ ((k >> 2) & 2u);
    const uint32_t e = k & 3u;
    const uint32_t f = ((e & 1u) * 6u) ^ ((e >> 1) * 10u);  // 0, 6, 10, 12
    return f & (uint32_t)(CHN - 1);
}

template <int BM, int BN, int BK, int WM, int WN, int STAGES>
struct PipeCfg {
    static constexpr int NW = WM * WN;        // waves
    static constexpr int NT = kWave * NW;     // threads
    static constexpr int CHA = BK / 8;        // 16-byte chunks per A row
    static constexpr int CHN = BN / 8;        // 16-byte chunks per B row
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    static constexpr int TM = WTM / 32, TN = WTN / 32;
    static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BK * BN * 2;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
    static constexpr int A_COPIES = A_BYTES / 1024;  // wave-wide 1 KiB copies per stage
    static constexpr int B_COPIES = B_BYTES / 1024;
    static constexpr int A_PER = A_COPIES / NW;      // per wave
    static constexpr int B_PER = B_COPIES / NW;
    static constexpr int LOADS = A_PER + B_PER;      // vmem ops per wave per stage

    static_assert(BK == 32 || BK == 64, "BK");
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile");
    static_assert(CHN >= 8, "B rows of at least 128 bytes");
    static_assert(A_COPIES % NW == 0 && B_COPIES % NW == 0, "copies split evenly over waves");
    static_assert(STAGES >= 2, "stages");
    static_assert(LDS_BYTES <= 163840, "gfx950 LDS per workgroup");
};

template <int BM, int BN, int BK, int WM, int WN, int STAGES>
__global__ void __launch_bounds__(kWave * WM * WN)
gemm_scale_relu_pipe_kernel(Problem p)
{
    using T = PipeCfg<BM, BN, BK, WM, WN, STAGES>;
    constexpr int NW = T::NW, CHA = T::CHA, CHN = T::CHN, TM = T::TM, TN = T::TN;

    __shared__ __attribute__((aligned(1024))) uint8_t smem[T::LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;

    int tm, tn;
    tile_of(blockIdx.x, gridDim.x, p, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    const i32x4 ra = raw_rsrc(p.A, (uint32_t)p.M * (uint32_t)p.K * 2u);
    const i32x4 rb = raw_rsrc(p.B, (uint32_t)p.K * (uint32_t)p.N * 2u);
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.C, (uint32_t)p.M * (uint32_t)p.N * 2u);
    const uint32_t lds0 = lds_address(smem);

    // ---- copy plan: this lane's source chunk for each of its wave's copies -
    // A copy j covers LDS chunk positions 64j..64j+63 of the A region:
    // position P -> row P / CHA, physical chunk P % CHA (= lane % CHA).
    uint32_t a_off[T::A_PER];  // byte offset of row start + chunk, without k0
    int a_k[T::A_PER];         // first k of the chunk (relative to k0)
    bool a_ok[T::A_PER];
#pragma unroll
    for (int i = 0; i < T::A_PER; ++i) {
        const int j = wave + i * NW;
        const int P = 64 * j + lane;
        const int r = P / CHA;
        const int c = (P % CHA) ^ (int)swz_a<CHA>(r);
        const int m = m0 + r;
        a_ok[i] = m < p.M;
        a_k[i] = 8 * c;
        a_off[i] = ((uint32_t)m * (uint32_t)p.K + (uint32_t)(8 * c)) * 2u;
    }
    // B copy j: position P -> row k = P / CHN, physical chunk P % CHN.
    uint32_t b_off[T::B_PER];  // byte offset of column chunk within a row (plus row k * N)
    int b_k[T::B_PER];
    bool b_ok[T::B_PER];
#pragma unroll
    for (int i = 0; i < T::B_PER; ++i) {
        const int j = wave + i * NW;
        const int P = 64 * j + lane;
        const int k = P / CHN;
        const int c = (P % CHN) ^ (int)swz_b<CHN>(k);
        const int n = n0 + 8 * c;
        b_ok[i] = n < p.N;
        b_k[i] = k;
        b_off[i] = ((uint32_t)k * (uint32_t)p.N + (uint32_t)n) * 2u;
    }

    auto issue = [&](int stage, int k0) {
        const uint32_t As = lds0 + stage * T::STAGE_BYTES;
        const uint32_t Bs = As + T::A_BYTES;
#pragma unroll
        for (int i = 0; i < T::A_PER; ++i) {
            const bool ok = a_ok[i] & (k0 + a_k[i] < p.K);
            const uint32_t off = ok ? a_off[i] + (uint32_t)k0 * 2u : kOutOfRange;
            copy16_to_lds(ra, off, As + (wave + i * NW) * 1024);
        }
#pragma unroll
        for (int i = 0; i < T::B_PER; ++i) {
            const bool ok = b_ok[i] & (k0 + b_k[i] < p.K);
            const uint32_t off = ok ? b_off[i] + (uint32_t)k0 * (uint32_t)p.N * 2u : kOutOfRange;
            copy16_to_lds(rb, off, Bs + (wave + i * NW) * 1024);
        }
    };

    // ---- fragment read plan ------------------------------------------------
    // A^T operand (32x32x16, second operand): lane l reads row (l % 32) of its
    // 32-row block, chunk 2*ks + l/32.
    const uint32_t frow = lane & 31, fhi = lane >> 5;
    uint32_t y_row[TM], y_sw[TM];
#pragma unroll
    for (int b = 0; b < TM; ++b) {
        const uint32_t r = wm * T::WTM + b * 32 + frow;
        y_row[b] = r * (BK * 2);
        y_sw[b] = swz_a<CHA>(r);
    }
    // B^T operand (first operand) through the transpose read: 16-lane group
    // G = l/16, i = l%16, e = i/4, q = i%4; source row 16*ks + 8*(G/2) + 4*rd + e,
    // source columns (block n) + 16*(G%2) + 4q .. +3.
    const uint32_t G = lane >> 4, li = lane & 15, e4 = li >> 2, q4 = li & 3;
    uint32_t x_chunk[TN];
#pragma unroll
    for (int a = 0; a < TN; ++a) x_chunk[a] = (wn * T::WTN + a * 32 + 16 * (G & 1)) / 8 + (q4 >> 1);
    const uint32_t x_half = (q4 & 1) * 8;
    const uint32_t x_k = 8 * (G >> 1) + e4;  // row within a 16-k substep, read 0

    f32x16 acc[TN][TM];
#pragma unroll
    for (int a = 0; a < TN; ++a)
#pragma unroll
        for (int b = 0; b < TM; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

    const int ksteps = (p.K + BK - 1) / BK;

    // prologue: the first STAGES-1 steps
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
        if (s < ksteps) issue(s, s * BK);

    for (int t = 0; t < ksteps; ++t) {
        // copies of step t are the oldest outstanding ones of this wave
        const int ahead = min(STAGES - 2, ksteps - 1 - t);  // later steps already issued
        if (ahead == STAGES - 2) wait_vmcnt<T::LOADS * (STAGES - 2)>();
        else wait_vmcnt_dyn(T::LOADS * ahead);
        lds_barrier();
        if (t + STAGES - 1 < ksteps) issue((t + STAGES - 1) % STAGES, (t + STAGES - 1) * BK);

        const uint8_t* As = smem + (t % STAGES) * T::STAGE_BYTES;
        const uint8_t* Bs = As + T::A_BYTES;
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            half8 xf[TN], yf[TM];
            const uint32_t c = 2 * ks + fhi;
#pragma unroll
            for (int b = 0; b < TM; ++b)
                yf[b] = __builtin_bit_cast(half8, *(const u32x4*)(As + y_row[b] + ((c ^ y_sw[b]) << 4)));
#pragma unroll
            for (int a = 0; a < TN; ++a) {
                v4i16 lo, hi;
                {
                    const uint32_t k = 16 * ks + x_k;
                    lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_v4i16*)(Bs + k * (BN * 2) + ((x_chunk[a] ^ swz_b<CHN>(k)) << 4) + x_half));
                }
                {
                    const uint32_t k = 16 * ks + x_k + 4;
                    hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_v4i16*)(Bs + k * (BN * 2) + ((x_chunk[a] ^ swz_b<CHN>(k)) << 4) + x_half));
                }
                xf[a] = __builtin_bit_cast(half8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
#pragma unroll
            for (int a = 0; a < TN; ++a)
#pragma unroll
                for (int b = 0; b < TM; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(xf[a], yf[b], acc[a][b], 0, 0, 0);
        }
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
