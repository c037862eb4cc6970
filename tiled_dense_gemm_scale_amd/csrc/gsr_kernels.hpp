// gsr_kernels.hpp -- gfx950 kernels for C = ReLU(alpha * A @ B), fp16 in/out,
// fp32 accumulation (PKUHPC scow-tutorial "Tutorial14", section 3 display
// formula; section 2's listing: one workgroup per output tile, a pipelined K
// loop of global->shared copies and tile products, the scale and max(., 0) on
// the accumulator fragment, one store).
//
// The CDNA4 form of that design:
//  * one workgroup per BM x BN tile of C, launched on a 1-D grid whose ids are
//    regrouped so that the eight XCDs each get a compact block of tiles
//    (their L2s are private) and tiles inside a block share A and B panels;
//  * K is walked in BK = 64 steps through a ring of LDS buffers.  The loads
//    for step t+1 are issued into registers before the MFMAs of step t, and
//    written to the other LDS buffer after them, so global latency hides
//    behind the math and each step needs one barrier;
//  * loads are raw buffer loads: out-of-range offsets return zero, which is
//    the ragged-edge rule (missing A/B elements contribute nothing), and
//    out-of-range buffer stores are dropped (nothing outside C is written);
//  * B arrives N-contiguous but an MFMA operand wants 8 K-contiguous values
//    per lane, so each thread loads an 8x8 block of B, transposes it in
//    registers with byte permutes and writes K-contiguous rows to LDS.  Both
//    LDS tiles are then [rows][BK] with 16-byte chunks XOR-swizzled by row,
//    which keeps the 128-bit writes and the 128-bit fragment reads free of
//    bank conflicts;
//  * the MFMA runs with B^T as its first operand and A^T as its second, so
//    the 32x32 accumulator block lands with four consecutive n per lane: the
//    epilogue scales, clamps at zero, converts with round-to-nearest-even and
//    stores 8 bytes per lane.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace gsr {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Any byte offset at or past a buffer's num_records reads as zero and is not
// written; every matrix is below 2^31 bytes, so this one always is.
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kWave = 64;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes)
{
    // flags word: the raw-buffer data format used on gfx9-family parts
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// 16-byte chunk c of LDS row r lives at chunk c ^ swz(r) (8 chunks per row).
__device__ __forceinline__ uint32_t swz(uint32_t r) { return (r ^ (r >> 3)) & 7u; }

// Eight consecutive fp16 values starting at element offset `elem`; the first
// `nvalid` of them exist (0..8).  The vector form needs nvalid in {0, 8} and
// a 16-byte aligned address; the element form loads the values one by one,
// each at its own (2-byte aligned) address.
template <bool VEC>
__device__ __forceinline__ u32x4 load8(__amdgpu_buffer_rsrc_t rs, uint32_t elem, int nvalid)
{
    if constexpr (VEC) {
        const uint32_t off = (nvalid > 0) ? elem * 2u : kOutOfRange;
        return __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
    } else {
        uint32_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t off = (e < nvalid) ? (elem + e) * 2u : kOutOfRange;
            h[e] = __builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, 0);
        }
        u32x4 v;
        v[0] = h[0] | (h[1] << 16);
        v[1] = h[2] | (h[3] << 16);
        v[2] = h[4] | (h[5] << 16);
        v[3] = h[6] | (h[7] << 16);
        return v;
    }
}

// load8 for the element-wise path with the operand's load unit U (16, 8, 4
// or 2 bytes).  Every row of the operand starts on a multiple of the unit and
// so does the end of the matrix, and a chunk starts on a multiple of 16 bytes
// from its row, so each load is naturally aligned and lies wholly inside or
// wholly outside the records.  Loads that hold no valid value are not issued;
// values past `nvalid` inside a load (the next row's) are cleared.
template <int U>
__device__ __forceinline__ u32x4 load8_unit(__amdgpu_buffer_rsrc_t rs, uint32_t elem, int nvalid)
{
    if constexpr (U == 16) {
        return load8<true>(rs, elem, nvalid);  // nvalid is 0 or 8 with this unit
    } else if constexpr (U == 2) {
        return load8<false>(rs, elem, nvalid);
    } else {
        const uint32_t off = elem * 2u;
        u32x4 v;
        if constexpr (U == 8) {
            const u32x2 lo = __builtin_amdgcn_raw_buffer_load_b64(rs, nvalid > 0 ? off : kOutOfRange, 0, 0);
            const u32x2 hi = __builtin_amdgcn_raw_buffer_load_b64(rs, nvalid > 4 ? off + 8u : kOutOfRange, 0, 0);
            v = u32x4{lo[0], lo[1], hi[0], hi[1]};
        } else {
            static_assert(U == 4, "load units of 16, 8, 4 or 2 bytes");
#pragma unroll
            for (int i = 0; i < 4; ++i)
                v[i] = __builtin_amdgcn_raw_buffer_load_b32(rs, nvalid > 2 * i ? off + 4u * (uint32_t)i : kOutOfRange, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (2 * i >= nvalid) v[i] = 0u;
            else if (2 * i + 1 >= nvalid) v[i] &= 0xffffu;
        }
        return v;
    }
}

// lo halves of x and y -> one dword (x low), hi halves likewise
__device__ __forceinline__ uint32_t pack_lo(uint32_t x, uint32_t y) { return __builtin_amdgcn_perm(y, x, 0x05040100u); }
__device__ __forceinline__ uint32_t pack_hi(uint32_t x, uint32_t y) { return __builtin_amdgcn_perm(y, x, 0x07060302u); }

// In: r[i] = 8 fp16 of row i (columns 0..7).  Out: o[j] = 8 fp16 of column j
// (rows 0..7).
__device__ __forceinline__ void transpose8x8(const u32x4 (&r)[8], u32x4 (&o)[8])
{
#pragma unroll
    for (int e = 0; e < 4; ++e) {      // row pair (2e, 2e+1) -> dword e of every output
#pragma unroll
        for (int d = 0; d < 4; ++d) {  // dword d of a row holds columns 2d, 2d+1
            o[2 * d][e] = pack_lo(r[2 * e][d], r[2 * e + 1][d]);
            o[2 * d + 1][e] = pack_hi(r[2 * e][d], r[2 * e + 1][d]);
        }
    }
}

struct Problem {
    const uint16_t* A;
    const uint16_t* B;
    uint16_t* C;
    const uint16_t* bias;  // N fp16 values, or null
    int M, N, K;
    float alpha;
    int act;               // kActRelu, kActGelu or kActNone
    int tiles_m, tiles_n;
    int group_m;
    int xcd_remap;
    // the element-wise kernel's load unit per operand, in bytes (16, 8, 4 or
    // 2): the largest power of two up to 16 that divides both the operand's
    // address and its row length in bytes (2K for A, 2N for B)
    int unit_a, unit_b;
    // the vector kernels' store unit for C, in bytes (16, 8, 4 or 2): the
    // largest power of two up to 16 dividing C's address (their rows of C are
    // 2N bytes apart, a multiple of 16)
    int unit_c;
    // K split across workgroups (the copy-wave K-split kernels with a
    // workspace): ksplit parts of kchunk K values each (a multiple of the
    // kernel's K-step; the last part ends at K), the parts' fp32 sums and the
    // tiles' arrival counters in the caller's workspace.  ksplit 1: none.
    int ksplit, kchunk;
    float* ws_part;
    uint32_t* ws_count;
};

// Eight outputs (16 bytes) at byte offset `off` of C, a multiple of 16 from
// C's start, written in stores of the launch's unit for C (U = 16, 8, 4 or 2
// bytes), so each store is naturally aligned.  An out-of-range offset
// (kOutOfRange and up) drops every part.  AUX is the cache policy.
template <int U, int AUX>
__device__ __forceinline__ void store16_unit(u32x4 v, __amdgpu_buffer_rsrc_t rc, uint32_t off)
{
    if constexpr (U == 16) {
        __builtin_amdgcn_raw_buffer_store_b128(v, rc, off, 0, AUX);
    } else if constexpr (U == 8) {
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{v[0], v[1]}, rc, off, 0, AUX);
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{v[2], v[3]}, rc, off + 8u, 0, AUX);
    } else if constexpr (U == 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) __builtin_amdgcn_raw_buffer_store_b32(v[i], rc, off + 4u * (uint32_t)i, 0, AUX);
    } else {
        static_assert(U == 2, "store units of 16, 8, 4 or 2 bytes");
#pragma unroll
        for (int i = 0; i < 8; ++i)
            __builtin_amdgcn_raw_buffer_store_b16((uint16_t)((i & 1) ? (v[i >> 1] >> 16) : (v[i >> 1] & 0xffffu)), rc,
                                                  off + 2u * (uint32_t)i, 0, AUX);
    }
}

// f(integral_constant<int, U>) for the launch's store unit: one uniform
// branch per store loop, each loop compiled for its unit.
template <class F>
__device__ __forceinline__ void with_store_unit(int unit, F&& f)
{
    if (unit == 16) f(std::integral_constant<int, 16>{});
    else if (unit == 8) f(std::integral_constant<int, 8>{});
    else if (unit == 4) f(std::integral_constant<int, 4>{});
    else f(std::integral_constant<int, 2>{});
}

// ---- epilogue -----------------------------------------------------------
// The tutorial's epilogue is v = alpha * acc, max(v, 0), narrow.  The
// epilogue variants (the aikraft.ru TileLang guide, section 4, GEMM + Bias +
// GELU) add one fp16 bias value per output column after the scale and apply
// ReLU, the tanh-form GELU or nothing: v = act(alpha * acc + bias[n]).
enum : int { kActRelu = 0, kActGelu = 1, kActNone = 2 };

// GELU, tanh form: y/2 (1 + tanh(u)) = y / (1 + exp(-2u)) with
// u = sqrt(2/pi) (y + 0.044715 y^3), evaluated with the hardware base-2
// exponential and reciprocal (about 1 ulp each, far below the fp16 output
// rounding).  exp(-2u) overflowing to +inf (very negative y) gives -0,
// underflowing to 0 (large y) gives y.
__device__ __forceinline__ float gelu_tanh(float y)
{
    // -2 * sqrt(2/pi) * log2(e), so that exp(-2u) = 2^(t * (y + 0.044715 y^3))
    constexpr float t = -2.0f * 0.7978845608028654f * 1.4426950408889634f;
    const float e = __builtin_amdgcn_exp2f(t * (y + 0.044715f * (y * y * y)));
    return y * __builtin_amdgcn_rcpf(1.0f + e);
}

__device__ __forceinline__ float activate(float y, int act)
{
    if (act == kActRelu) return y > 0.0f ? y : 0.0f;
    if (act == kActGelu) return gelu_tanh(y);
    return y;
}

// True when the epilogue is the tutorial's (no bias, ReLU): kernels keep a
// separate loop for it.
__device__ __forceinline__ bool plain_epilogue(const Problem& p) { return p.bias == nullptr && p.act == kActRelu; }

// The bias of columns n..n+3 (n a multiple of 4, bias 8-byte aligned, N a
// multiple of 8: the four are all inside or all outside; outside reads 0).
__device__ __forceinline__ f32x4 bias4(__amdgpu_buffer_rsrc_t rbias, int n)
{
    const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(rbias, (uint32_t)n * 2u, 0, 0);
    const half4 h = __builtin_bit_cast(half4, w);
    f32x4 f;
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = (float)h[i];
    return f;
}

// The bias of column n alone (any alignment; outside reads 0).
__device__ __forceinline__ float bias1(__amdgpu_buffer_rsrc_t rbias, int n)
{
    const uint16_t b = __builtin_amdgcn_raw_buffer_load_b16(rbias, (uint32_t)n * 2u, 0, 0);
    return (float)__builtin_bit_cast(_Float16, b);
}

// A descriptor over the bias (zero records when there is none).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t bias_rsrc(const Problem& p)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.bias), (short)0,
                                             p.bias ? p.N * 2 : 0, 0x00020000);
}

// The activation as a compile-time choice, so an epilogue loop carries no
// per-element branch.
template <int ACT>
__device__ __forceinline__ float activate_t(float y)
{
    if constexpr (ACT == kActRelu) return y > 0.0f ? y : 0.0f;
    else if constexpr (ACT == kActGelu) return gelu_tanh(y);
    else return y;
}

// act(alpha * s + b) for four outputs, narrowed to fp16 (round to nearest even).
template <int ACT>
__device__ __forceinline__ half4 epilogue4(f32x4 s, float alpha, f32x4 b)
{
    half4 h;
#pragma unroll
    for (int i = 0; i < 4; ++i) h[i] = (_Float16)activate_t<ACT>(s[i] * alpha + b[i]);
    return h;
}

// Runs f(std::integral_constant<int, ACT>) for the run-time activation code:
// one uniform branch per epilogue instead of one per element.
template <class F>
__device__ __forceinline__ void with_activation(int act, F&& f)
{
    if (act == kActGelu) f(std::integral_constant<int, kActGelu>{});
    else if (act == kActNone) f(std::integral_constant<int, kActNone>{});
    else f(std::integral_constant<int, kActRelu>{});
}

// Workgroup id -> (tile row, tile column).
//  xcd_remap 0: grouped order on the workgroup ids as dispatched.
//  xcd_remap 1: the same on ids regrouped so that each XCD gets a contiguous
//    range of them (consecutive tiles share an XCD's L2).
//  xcd_remap 2: chip rounds of 16 x 16 tiles, for grids that divide into
//    them (otherwise as 1): workgroups go to the 8 XCDs round-robin and an
//    XCD's 32 CUs run its workgroups 32 at a time, so slot s of XCD x runs in
//    round s / 32; in every round the chip covers one 16 x 16 block of tiles,
//    XCD x a 4 x 8 part of it (rows 4 (x / 2) .., columns 8 (x % 2) ..).
//    Each XCD's L2 still needs 4 A and 8 B panels per round, as in order 1,
//    but the chip as a whole needs 16 + 16 panels from HBM per round instead
//    of 32 + 8 (in order 1 every XCD holds its own tile rows).  group_m is
//    not used.  At 16384^3 with 256 x 256 tiles this measured 0.9 % faster
//    than order 1 (interleaved timings on one MI355X).
__device__ __forceinline__ void tile_of(int pid, int nwg, const Problem& p, int& tm, int& tn)
{
    if (p.xcd_remap == 2 && (p.tiles_m & 15) == 0 && (p.tiles_n & 15) == 0) {
        const int x = pid & 7, s = pid >> 3;  // XCD, slot in its dispatch order
        const int r = s >> 5, j = s & 31;     // round, tile of the round on this XCD
        const int per_row = p.tiles_n >> 4;   // 16 x 16 blocks per block row
        tm = (r / per_row) * 16 + (x >> 1) * 4 + (j & 3);
        tn = (r % per_row) * 16 + (x & 1) * 8 + (j >> 2);
        return;
    }
    if (p.xcd_remap) {
        // Workgroups are handed to the 8 XCDs round-robin: give XCD x a
        // contiguous range of logical ids instead.
        const int q = nwg >> 3, r = nwg & 7;
        const int x = pid & 7, idx = pid >> 3;
        pid = (x < r) ? x * (q + 1) + idx : r * (q + 1) + (x - r) * q + idx;
    }
    const int per_group = p.group_m * p.tiles_n;
    const int g = pid / per_group;
    const int first_m = g * p.group_m;
    const int gs = min(p.tiles_m - first_m, p.group_m);
    const int within = pid - g * per_group;
    tm = first_m + within % gs;
    tn = within / gs;
}

template <int BM, int BN, int BK, int WM, int WN, bool VEC>
struct TileKernel {
    static constexpr int NT = kWave * WM * WN;  // threads per workgroup
    static constexpr int CH = BK / 8;           // 16-byte chunks per LDS row
    static constexpr int WTM = BM / WM;         // wave tile rows (m)
    static constexpr int WTN = BN / WN;         // wave tile cols (n)
    static constexpr int TM = WTM / 32;         // 32x32 MFMA blocks per wave, m
    static constexpr int TN = WTN / 32;         // ... n
    static constexpr int A_BYTES = BM * BK * 2;
    static constexpr int B_BYTES = BN * BK * 2;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int LDS_BYTES = 2 * STAGE_BYTES;
    static constexpr int A_CHUNKS = BM * CH;               // 16-byte chunks of an A tile
    static constexpr int A_PER = A_CHUNKS / NT;            // per thread
    static constexpr int B_BLOCKS = (BK / 8) * (BN / 8);   // 8x8 blocks of a B tile
    static constexpr int B_PER = (B_BLOCKS + NT - 1) / NT; // per thread (last may be partial)

    static_assert(BK == 64, "the LDS swizzle assumes 8 chunks per row");
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32x32");
    static_assert(A_CHUNKS % NT == 0 && NT % CH == 0, "A tile must split evenly over threads");
    static_assert(LDS_BYTES <= 163840, "LDS budget of one workgroup on gfx950");
};

template <int BM, int BN, int BK, int WM, int WN, bool VEC>
__global__ void __launch_bounds__(kWave * WM * WN)
gemm_scale_relu_kernel(Problem p)
{
    using T = TileKernel<BM, BN, BK, WM, WN, VEC>;
    constexpr int NT = T::NT, CH = T::CH, TM = T::TM, TN = T::TN;

    __shared__ __attribute__((aligned(16))) uint8_t smem[T::LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

    int tm, tn;
    tile_of(blockIdx.x, gridDim.x, p, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    const uint32_t a_bytes = (uint32_t)p.M * (uint32_t)p.K * 2u;
    const uint32_t b_bytes = (uint32_t)p.K * (uint32_t)p.N * 2u;
    const uint32_t c_bytes = (uint32_t)p.M * (uint32_t)p.N * 2u;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A, a_bytes);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.B, b_bytes);
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.C, c_bytes);

    // ---- this thread's share of each global -> LDS copy -------------------
    // A: chunk ids tid + i*NT; since NT is a multiple of CH the chunk column is
    // the same for every i.
    const int a_kc = tid % CH;
    const int a_r0 = tid / CH;
    constexpr int A_ROW_STEP = NT / CH;
    // B: 8x8 block ids tid + i*NT, block (kb, nb) = rows kb*8.., cols nb*8..
    constexpr int NB8 = BN / 8;

    u32x4 areg[T::A_PER];
    u32x4 breg[T::B_PER][8];

    // On the element-wise path each operand is read in the widest unit its
    // alignment allows (p.unit_a, p.unit_b); the unit is picked once per
    // K-step (a uniform branch on a kernel argument) for a copy of the load
    // loop compiled for it, so the loads of a step still issue back to back.
    // The vector path reads 16-byte units throughout.
    auto load_a = [&](auto unit_tag, int k0) {
        constexpr int U = decltype(unit_tag)::value;
        const int kk = k0 + a_kc * 8;
        const int kval = min(max(p.K - kk, 0), 8);
#pragma unroll
        for (int i = 0; i < T::A_PER; ++i) {
            const int r = a_r0 + i * A_ROW_STEP;
            const int m = m0 + r;
            const int nv = (m < p.M) ? kval : 0;
            areg[i] = load8_unit<U>(ra, (uint32_t)m * (uint32_t)p.K + (uint32_t)kk, nv);
        }
    };
    auto load_b = [&](auto unit_tag, int k0) {
        constexpr int U = decltype(unit_tag)::value;
#pragma unroll
        for (int i = 0; i < T::B_PER; ++i) {
            const int blk = tid + i * NT;
            if (T::B_BLOCKS % NT == 0 || blk < T::B_BLOCKS) {
                const int kb = blk / NB8, nb = blk % NB8;
                const int n = n0 + nb * 8;
                const int nval = min(max(p.N - n, 0), 8);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int k = k0 + kb * 8 + j;
                    const int nv = (k < p.K) ? nval : 0;
                    breg[i][j] = load8_unit<U>(rb, (uint32_t)k * (uint32_t)p.N + (uint32_t)n, nv);
                }
            }
        }
    };
    using U16 = std::integral_constant<int, 16>;
    using U8 = std::integral_constant<int, 8>;
    using U4 = std::integral_constant<int, 4>;
    using U2 = std::integral_constant<int, 2>;
    auto with_unit = [&](int unit, auto&& f) {
        if constexpr (VEC) {
            f(U16{});
        } else {
            if (unit == 16) f(U16{});
            else if (unit == 8) f(U8{});
            else if (unit == 4) f(U4{});
            else f(U2{});
        }
    };
    auto load_tile = [&](int k0) {
        with_unit(p.unit_a, [&](auto u) { load_a(u, k0); });
        with_unit(p.unit_b, [&](auto u) { load_b(u, k0); });
    };

    auto store_tile = [&](int stage) {
        uint8_t* As = smem + stage * T::STAGE_BYTES;
        uint8_t* Bs = As + T::A_BYTES;
#pragma unroll
        for (int i = 0; i < T::A_PER; ++i) {
            const uint32_t r = a_r0 + i * A_ROW_STEP;
            *(u32x4*)(As + r * (BK * 2) + ((a_kc ^ swz(r)) << 4)) = areg[i];
        }
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
                    *(u32x4*)(Bs + r * (BK * 2) + ((kb ^ swz(r)) << 4)) = col[j];
                }
            }
        }
    };

    // ---- fragment addresses -----------------------------------------------
    // MFMA 32x32x16: lane l supplies row (l % 32) of its 32-row operand block
    // and the 8 consecutive k of chunk (2*s + l/32) in k-substep s.
    const uint32_t frow = lane & 31;
    const uint32_t fhi = lane >> 5;
    uint32_t xoff[TN], xsw[TN], yoff[TM], ysw[TM];
#pragma unroll
    for (int t = 0; t < TN; ++t) {
        const uint32_t r = wn * T::WTN + t * 32 + frow;
        xoff[t] = T::A_BYTES + r * (BK * 2);
        xsw[t] = swz(r);
    }
#pragma unroll
    for (int t = 0; t < TM; ++t) {
        const uint32_t r = wm * T::WTM + t * 32 + frow;
        yoff[t] = r * (BK * 2);
        ysw[t] = swz(r);
    }

    f32x16 acc[TN][TM];
#pragma unroll
    for (int a = 0; a < TN; ++a)
#pragma unroll
        for (int b = 0; b < TM; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

    const int ksteps = (p.K + BK - 1) / BK;

    load_tile(0);
    store_tile(0);
    __syncthreads();

    for (int t = 0; t < ksteps; ++t) {
        const int cur = t & 1;
        const bool more = (t + 1) < ksteps;
        if (more) load_tile((t + 1) * BK);

        const uint8_t* base = smem + cur * T::STAGE_BYTES;
#pragma unroll
        for (int s = 0; s < BK / 16; ++s) {
            const uint32_t c = 2 * s + fhi;
            half8 xf[TN], yf[TM];
#pragma unroll
            for (int a = 0; a < TN; ++a)
                xf[a] = __builtin_bit_cast(half8, *(const u32x4*)(base + xoff[a] + ((c ^ xsw[a]) << 4)));
#pragma unroll
            for (int b = 0; b < TM; ++b)
                yf[b] = __builtin_bit_cast(half8, *(const u32x4*)(base + yoff[b] + ((c ^ ysw[b]) << 4)));
#pragma unroll
            for (int a = 0; a < TN; ++a)
#pragma unroll
                for (int b = 0; b < TM; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(xf[a], yf[b], acc[a][b], 0, 0, 0);
        }

        if (more) store_tile(cur ^ 1);
        __syncthreads();
    }

    // ---- epilogue: scale, clamp at zero, narrow, store ---------------------
    // Accumulator block (a, b): lane l holds m = l % 32 and, in register
    // 4g + i, n = 8g + 4*(l/32) + i.
    const float alpha = p.alpha;
    // four outputs n..n+3 of row m: the element path writes them with the
    // widest naturally aligned stores their address allows (one of 8 bytes,
    // two of 4, or 2 + 4 + 2), and one by one at the edge of C
    const uint32_t c_align = (uint32_t)(uintptr_t)p.C & 7u;
    auto store4 = [&](int m, int n, half4 h) {
        const u32x2 w = __builtin_bit_cast(u32x2, h);
        const uint32_t elem = (uint32_t)m * (uint32_t)p.N + (uint32_t)n;
        if constexpr (VEC) {
            const uint32_t off = ((m < p.M) & (n < p.N)) ? elem * 2u : kOutOfRange;
            __builtin_amdgcn_raw_buffer_store_b64(w, rc, off, 0, 0);
        } else {
            const uint32_t off = elem * 2u, al = (c_align + off) & 7u;
            if ((m < p.M) & (n + 3 < p.N)) {
                if (al == 0u) {
                    __builtin_amdgcn_raw_buffer_store_b64(w, rc, off, 0, 0);
                } else if (al == 4u) {
                    __builtin_amdgcn_raw_buffer_store_b32(w[0], rc, off, 0, 0);
                    __builtin_amdgcn_raw_buffer_store_b32(w[1], rc, off + 4u, 0, 0);
                } else {  // 2 mod 4: values 1 and 2 share an aligned dword
                    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(w[0] & 0xffffu), rc, off, 0, 0);
                    __builtin_amdgcn_raw_buffer_store_b32((w[0] >> 16) | (w[1] << 16), rc, off + 2u, 0, 0);
                    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(w[1] >> 16), rc, off + 6u, 0, 0);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t o = ((m < p.M) & (n + i < p.N)) ? (elem + i) * 2u : kOutOfRange;
                    const uint16_t hv = (uint16_t)((i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xffffu));
                    __builtin_amdgcn_raw_buffer_store_b16(hv, rc, o, 0, 0);
                }
            }
        }
    };
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
                    store4(m, n, h);
                }
            }
        }
    } else {
        // the bias of the lane's columns, all requested before the first use
        const __amdgpu_buffer_rsrc_t rbias = bias_rsrc(p);
        f32x4 bvs[TN][4];
#pragma unroll
        for (int a = 0; a < TN; ++a) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = n0 + wn * T::WTN + a * 32 + 8 * g + 4 * (int)fhi;
                if (p.bias == nullptr) {
                    bvs[a][g] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                } else if constexpr (VEC) {
                    bvs[a][g] = bias4(rbias, n);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) bvs[a][g][i] = (n + i < p.N) ? bias1(rbias, n + i) : 0.0f;
                }
            }
        }
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
                        store4(m, n, epilogue4<ACT>(sv, alpha, bv));
                    }
                }
            }
        });
    }
}

// K == 0: every output is the empty sum, so C[m,n] = act(alpha * 0 + bias[n])
// (+0 without a bias).
__global__ void __launch_bounds__(256) fill_epilogue_kernel(uint16_t* C, uint32_t M, uint32_t N,
                                                            const uint16_t* bias, float alpha, int act)
{
    const uint32_t count = M * N;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(C, count * 2u);
    for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < count; i += gridDim.x * 256u) {
        uint16_t out = 0;
        if (bias != nullptr || act != kActRelu) {
            const float b = bias ? (float)__builtin_bit_cast(_Float16, bias[i % N]) : 0.0f;
            out = __builtin_bit_cast(uint16_t, (_Float16)activate(0.0f * alpha + b, act));
        }
        __builtin_amdgcn_raw_buffer_store_b16(out, rc, i * 2u, 0, 0);
    }
}

}  // namespace gsr
