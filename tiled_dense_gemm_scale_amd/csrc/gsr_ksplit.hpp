// gsr_ksplit.hpp -- small-tile 128-bit path of C = ReLU(alpha * A @ B) for
// shapes with few output tiles (e.g. 1024^3 gives 256 tiles of 64x64, one per
// CU) and for skinny shapes.
//
// With a 64x64 tile split over four waves by output, each wave gets a single
// 32x32 MFMA per 16-k substep, and every K-step becomes a chain of LDS
// latency, one MFMA and a barrier.  Here the four waves split K instead: each
// K-step covers BK = 128 (eight 16-k substeps) and wave w computes substeps w
// and w+4 for the whole BM x BN tile, so a wave issues 8..16 MFMAs per step
// and the operand bytes each wave reads per MFMA halve.
//  * A and B are copied global -> LDS by the buffer unit (buffer_load ... lds)
//    into a ring of STAGES buffers kept STAGES-1 steps ahead; out-of-range
//    chunks read as zero (ragged M, N, K).
//  * A lands as [BM][128] rows (16-byte chunks XOR-swizzled by row), read with
//    128-bit LDS reads; B lands as [128][BN] rows and is read with the gfx950
//    transpose read, which hands each lane four K-consecutive values of one
//    column.
//  * The operand reads of step t are issued right after the barrier that
//    publishes step t, and the MFMAs of step t-1 run behind them.
//  * At the end the four partial tiles are summed through LDS (KsSum below):
//    each thread sums one row's eight consecutive outputs over the waves,
//    applies the epilogue (scale, clamp at zero, round to fp16; or scale,
//    bias, activation) and writes them with one 16-byte store.
#pragma once

#include "gsr_pipeline.hpp"

namespace gsr {

template <int BM, int BN, int STAGES>
struct KsCfg {
    static constexpr int BK = 128, NW = 4, NT = kWave * NW;
    static constexpr int CHA = BK / 8;   // 16 chunks per A row (256 bytes)
    static constexpr int CHN = BN / 8;   // chunks per B row
    static constexpr int TM = BM / 32, TN = BN / 32;
    static constexpr int NB = TM * TN;  // accumulator blocks per wave
    static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BK * BN * 2;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int RED_BYTES = NW * NB * 4 * 1024;  // partial tiles for the reduction
    static constexpr int LDS_BYTES = (STAGES * STAGE_BYTES > RED_BYTES) ? STAGES * STAGE_BYTES : RED_BYTES;
    static constexpr int A_PER = A_BYTES / 1024 / NW;  // copies per wave per step
    static constexpr int B_PER = B_BYTES / 1024 / NW;
    static constexpr int LOADS = A_PER + B_PER;
    static_assert(BM % 32 == 0 && BN % 32 == 0 && CHN >= 4, "tile");
    static_assert((A_BYTES / 1024) % NW == 0 && (B_BYTES / 1024) % NW == 0, "copies split over waves");
    static_assert(STAGES >= 2 && LDS_BYTES <= 163840, "LDS");
};

// 16-chunk (256-byte) A rows: chunk c of row r sits at c ^ f(r); any 16
// consecutive rows read at one logical chunk hit 16 distinct positions.
__device__ __forceinline__ uint32_t swz_a16(uint32_t r) { return (r ^ (r >> 4)) & 15u; }

// ---- the cross-wave sum of the K-split partial tiles ------------------------
// Each of the NW waves writes its BM x BN fp32 partial tile to LDS as
// row-major rows of BN*4 bytes whose 16-byte chunks are XOR-swizzled by row
// (chunk c of row m sits at c ^ (m mod chunks-per-row)): the writes from the
// MFMA lane layout (16 lanes = 16 rows at distinct chunks) and the row reads
// (8 lanes = 8 consecutive chunks of one row; the next 8 lanes read the next
// row, whose swizzle lands on the other half of the banks) do not conflict.
// A sum unit is one row's eight consecutive outputs: its chunks are summed
// over the waves in wave order (the same order for every element), then the
// epilogue runs and one 16-byte store writes the unit.  Consecutive threads
// take consecutive units, so the stores of a wave cover whole rows.
template <int BM, int BN, int NW, int NT>
struct KsSum {
    static constexpr int QN = BN / 8;               // units per tile row
    static constexpr int UNITS = BM * QN;
    static constexpr int NU = (UNITS + NT - 1) / NT;  // units per thread
    static constexpr int CPR = BN / 4;              // 16-byte chunks per partial row
    static constexpr int PART_BYTES = BM * BN * 4;
    static constexpr int BYTES = NW * PART_BYTES;
    static_assert(BN % 32 == 0 && BM % 32 == 0, "tile");

    __device__ static uint32_t addr(int w, int m, int chunk)
    {
        return (uint32_t)(w * PART_BYTES + m * (BN * 4)) + ((uint32_t)(chunk ^ (m & (CPR - 1))) << 4);
    }

    // bias values of this thread's units (zeros where the epilogue has none)
    __device__ static void load_bias(const Problem& p, int tid, int n0, f32x4 (&bvs)[NU][2])
    {
        const __amdgpu_buffer_rsrc_t rbias = bias_rsrc(p);
        const bool load = !plain_epilogue(p) && p.bias != nullptr;
#pragma unroll
        for (int j = 0; j < NU; ++j) {
            const int u = tid + NT * j;
            const int n = n0 + 8 * (u % QN);
            const bool ok = load && u < UNITS;
            bvs[j][0] = ok ? bias4(rbias, n) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            bvs[j][1] = ok ? bias4(rbias, n + 4) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
    }

    // wave w's partial tile: MFMA block (a, b), registers 4g..4g+3 of lane l
    // hold row b*32 + l%32, columns a*32 + 8g + 4*(l/32) .. +3, i.e. fp32
    // chunk 8a + 2g + l/32 of that row
    template <int TN, int TM>
    __device__ static void write(uint8_t* smem, const f32x16 (&acc)[TN][TM], int w, int lane)
    {
        const int frow = lane & 31, fhi = lane >> 5;
#pragma unroll
        for (int a = 0; a < TN; ++a)
#pragma unroll
            for (int b = 0; b < TM; ++b)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const f32x16 av = acc[a][b];
                    f32x4 v;
                    if (g == 0) v = __builtin_shufflevector(av, av, 0, 1, 2, 3);
                    else if (g == 1) v = __builtin_shufflevector(av, av, 4, 5, 6, 7);
                    else if (g == 2) v = __builtin_shufflevector(av, av, 8, 9, 10, 11);
                    else v = __builtin_shufflevector(av, av, 12, 13, 14, 15);
                    *(f32x4*)(smem + addr(w, b * 32 + frow, 8 * a + 2 * g + fhi)) = v;
                }
    }

    // unit u's eight outputs summed over the waves' partial tiles, in wave
    // order, starting from +0
    struct Sums {
        f32x4 lo, hi;
    };
    __device__ static Sums unit_sum(const uint8_t* smem, int u)
    {
        const int mr = u / QN, q = u % QN;
        f32x4 lo[NW], hi[NW];
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            lo[w] = *(const f32x4*)(smem + addr(w, mr, 2 * q));
            hi[w] = *(const f32x4*)(smem + addr(w, mr, 2 * q + 1));
        }
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < NW; ++w) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                s0[i] += lo[w][i];
                s1[i] += hi[w][i];
            }
        }
        return Sums{s0, s1};
    }

    // the epilogue of one unit's eight sums and its store to C
    template <int ACT, int U>
    __device__ static void finish(const Problem& p, __amdgpu_buffer_rsrc_t rc, bool plain, f32x4 s0, f32x4 s1,
                                  const f32x4 (&bv)[2], int m, int n)
    {
        const float alpha = p.alpha;
        half4 h0, h1;
        if (plain) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float v0 = s0[i] * alpha, v1 = s1[i] * alpha;
                h0[i] = (_Float16)(v0 > 0.0f ? v0 : 0.0f);
                h1[i] = (_Float16)(v1 > 0.0f ? v1 : 0.0f);
            }
        } else {
            h0 = epilogue4<ACT>(s0, alpha, bv[0]);
            h1 = epilogue4<ACT>(s1, alpha, bv[1]);
        }
        const uint32_t off = ((m < p.M) & (n < p.N)) ? ((uint32_t)m * (uint32_t)p.N + (uint32_t)n) * 2u : kOutOfRange;
        const u32x2 w0 = __builtin_bit_cast(u32x2, h0), w1 = __builtin_bit_cast(u32x2, h1);
        store16_unit<U, 0>(u32x4{w0[0], w0[1], w1[0], w1[1]}, rc, off);
    }

    __device__ static void sum_store(const Problem& p, const uint8_t* smem, int tid, int m0, int n0,
                                     const f32x4 (&bvs)[NU][2])
    {
        const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.C, (uint32_t)p.M * (uint32_t)p.N * 2u);
        const bool plain = plain_epilogue(p);
        with_activation(p.act, [&](auto act_tag) {
            with_store_unit(p.unit_c, [&](auto unit_tag) {
                constexpr int ACT = decltype(act_tag)::value;
                constexpr int U = decltype(unit_tag)::value;
#pragma unroll
                for (int j = 0; j < NU; ++j) {
                    const int u = tid + NT * j;
                    if (UNITS % NT != 0 && u >= UNITS) break;
                    const Sums t = unit_sum(smem, u);
                    finish<ACT, U>(p, rc, plain, t.lo, t.hi, bvs[j], m0 + u / QN, n0 + 8 * (u % QN));
                }
            });
        });
    }

    // The same sum when the tile's K range is split over p.ksplit
    // workgroups (part `part` of tile `tile` here).  Each workgroup writes its
    // fp32 sums to its slot of the workspace's partial tiles and counts
    // itself in the tile's arrival counter; the workgroup that arrives last
    // adds the parts in part order (0, 1, ..., starting from +0, its own sums
    // standing in for its slot), so the result does not depend on the
    // arrival order, runs the epilogue, stores C and puts the counter back to
    // zero for the next call.  No workgroup waits for another.
    //
    // The workgroups of a tile may run on different XCDs, whose L2 caches
    // are not coherent with each other.  The partial sums are therefore
    // written and read with device-scope accesses (relaxed atomics at agent
    // scope: stores that write through the L2, loads that do not take a
    // possibly stale L2 line), each wave waits until its stores have
    // completed before the workgroup barrier that precedes the count, and the
    // last workgroup reads only after its count has returned.  Release and
    // acquire fences at agent scope would order the same accesses, but they
    // write back and invalidate the whole L2: timed with them, every
    // workgroup added about 0.2 us, serialised per XCD.
    __device__ static void split_sum_store(const Problem& p, const uint8_t* smem, int* flag, int tid, int m0, int n0,
                                           const f32x4 (&bvs)[NU][2], int tile, int part)
    {
        static_assert(NU == 1, "one sum unit per thread");
        const int tiles = p.tiles_m * p.tiles_n, parts = p.ksplit;
        const int u = tid;
        const int m = m0 + u / QN, n = n0 + 8 * (u % QN);
        const bool live = (UNITS % NT == 0 || u < UNITS) && (m < p.M) && (n < p.N);
        // the unit's eight sums of part g: four 64-bit words
        const size_t slot = (size_t)tile * (BM * BN) + (size_t)u * 8, stride = (size_t)tiles * (BM * BN);
        auto words = [&](int g) { return (uint64_t*)(p.ws_part + (slot + (size_t)g * stride)); };
        Sums own{};
        if (live) {
            own = unit_sum(smem, u);
            const u32x4 lo = __builtin_bit_cast(u32x4, own.lo), hi = __builtin_bit_cast(u32x4, own.hi);
            uint64_t* dst = words(part);
            const uint64_t w[4] = {lo[0] | (uint64_t)lo[1] << 32, lo[2] | (uint64_t)lo[3] << 32,
                                   hi[0] | (uint64_t)hi[1] << 32, hi[2] | (uint64_t)hi[3] << 32};
#pragma unroll
            for (int i = 0; i < 4; ++i) __hip_atomic_store(dst + i, w[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        wait_vmcnt<0>();  // this wave's partial sums have reached device scope
        __syncthreads();
        if (tid == 0) {
            const uint32_t before = __hip_atomic_fetch_add(p.ws_count + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            *flag = (int)(before == (uint32_t)(parts - 1));
        }
        __syncthreads();
        if (*flag == 0) return;

        f32x4 t0 = {0.f, 0.f, 0.f, 0.f}, t1 = {0.f, 0.f, 0.f, 0.f};
        if (live) {
            for (int g = 0; g < parts; ++g) {
                f32x4 v0 = own.lo, v1 = own.hi;
                if (g != part) {
                    const uint64_t* src = words(g);
                    uint64_t w[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) w[i] = __hip_atomic_load(src + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    v0 = __builtin_bit_cast(f32x4, u32x4{(uint32_t)w[0], (uint32_t)(w[0] >> 32), (uint32_t)w[1], (uint32_t)(w[1] >> 32)});
                    v1 = __builtin_bit_cast(f32x4, u32x4{(uint32_t)w[2], (uint32_t)(w[2] >> 32), (uint32_t)w[3], (uint32_t)(w[3] >> 32)});
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    t0[i] += v0[i];
                    t1[i] += v1[i];
                }
            }
        }
        const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.C, (uint32_t)p.M * (uint32_t)p.N * 2u);
        const bool plain = plain_epilogue(p);
        const f32x4 b0 = bvs[0][0], b1 = bvs[0][1];
        with_activation(p.act, [&](auto act_tag) {
            with_store_unit(p.unit_c, [&](auto unit_tag) {
                constexpr int ACT = decltype(act_tag)::value;
                constexpr int U = decltype(unit_tag)::value;
                const f32x4 bv[2] = {b0, b1};
                // a unit outside C gets an out-of-range offset and stores nothing
                finish<ACT, U>(p, rc, plain, t0, t1, bv, live ? m : p.M, n);
            });
        });
        if (tid == 0) __hip_atomic_store(p.ws_count + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
};

template <int BM, int BN, int STAGES>
__global__ void __launch_bounds__(256)
gemm_scale_relu_ksplit_kernel(Problem p)
{
    using T = KsCfg<BM, BN, STAGES>;
    constexpr int BK = T::BK, NW = T::NW, CHA = T::CHA, CHN = T::CHN, TM = T::TM, TN = T::TN;

    __shared__ __attribute__((aligned(1024))) uint8_t smem[T::LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    int tm, tn;
    tile_of(blockIdx.x, gridDim.x, p, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    const i32x4 ra = raw_rsrc(p.A, (uint32_t)p.M * (uint32_t)p.K * 2u);
    const i32x4 rb = raw_rsrc(p.B, (uint32_t)p.K * (uint32_t)p.N * 2u);
    const uint32_t lds0 = lds_address(smem);

    // ---- copy plan ------------------------------------------------------------
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
        a_off[i] = ((uint32_t)m * (uint32_t)p.K + (uint32_t)(8 * c)) * 2u;
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
        b_off[i] = ((uint32_t)k * (uint32_t)p.N + (uint32_t)n) * 2u;
    }
    auto issue = [&](int stage, int k0) {
        const uint32_t As = lds0 + stage * T::STAGE_BYTES;
        const uint32_t Bs = As + T::A_BYTES;
#pragma unroll
        for (int i = 0; i < T::A_PER; ++i) {
            const bool ok = a_ok[i] & (k0 + a_k[i] < p.K);
            copy16_to_lds(ra, ok ? a_off[i] + (uint32_t)k0 * 2u : kOutOfRange, As + (wave + i * NW) * 1024);
        }
#pragma unroll
        for (int i = 0; i < T::B_PER; ++i) {
            const bool ok = b_ok[i] & (k0 + b_k[i] < p.K);
            copy16_to_lds(rb, ok ? b_off[i] + (uint32_t)k0 * (uint32_t)p.N * 2u : kOutOfRange, Bs + (wave + i * NW) * 1024);
        }
    };

    // ---- operand reads: substeps ks = wave and wave + 4 of each step ---------
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

    // Two operand sets: the reads of step t fill set t & 1 while the MFMAs of
    // step t-1 use the other.  Both start as zeros so no path reads an
    // unwritten register.
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
    // iteration t: wait for step t's copies, publish them, refill the buffer
    // step t-1 used, read step t, multiply step t-1
    auto sync_and_refill = [&](int t, int ksteps) {
        const int ahead = min(STAGES - 2, ksteps - 1 - t);
        if (ahead == STAGES - 2) wait_vmcnt<T::LOADS * (STAGES - 2)>();
        else wait_vmcnt_dyn(T::LOADS * ahead);
        lds_barrier();
        if (t + STAGES - 1 < ksteps) issue((t + STAGES - 1) % STAGES, (t + STAGES - 1) * BK);
    };

    const int ksteps = (p.K + BK - 1) / BK;
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
        if (s < ksteps) issue(s, s * BK);

    int t = 0;
    for (; t + 1 < ksteps; t += 2) {
        sync_and_refill(t, ksteps);
        read_step(t % STAGES, xs0, ys0);
        if (t > 0) mma_step(xs1, ys1);
        sync_and_refill(t + 1, ksteps);
        read_step((t + 1) % STAGES, xs1, ys1);
        mma_step(xs0, ys0);
    }
    if (t < ksteps) {  // odd step count: one more even step
        sync_and_refill(t, ksteps);
        read_step(t % STAGES, xs0, ys0);
        if (t > 0) mma_step(xs1, ys1);
        mma_step(xs0, ys0);
    } else if (ksteps > 0) {
        mma_step(xs1, ys1);
    }

    // ---- sum the four partial tiles through LDS ---------------------------------
    // The variant's bias values are requested first, so their latency
    // overlaps the barrier and the partial-tile writes.
    using Sum = KsSum<BM, BN, NW, T::NT>;
    static_assert(Sum::BYTES <= T::LDS_BYTES, "partial tiles fit in LDS");
    f32x4 bvs[Sum::NU][2];
    Sum::load_bias(p, tid, n0, bvs);
    wait_vmcnt<0>();
    lds_barrier();  // every wave is done with the operand buffers
    Sum::write(smem, acc, wave, lane);
    lds_barrier();
    Sum::sum_store(p, smem, tid, m0, n0, bvs);
}

}  // namespace gsr
