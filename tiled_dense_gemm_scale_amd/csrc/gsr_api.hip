// gsr_api.hip -- host side of the C ABI declared in include/gsr.h: argument
// checks, device check, tile selection and the launch on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "gsr.h"
#include "gsr_kernels.hpp"
#include "gsr_pipeline.hpp"
#include "gsr_interleave.hpp"
#include "gsr_ksplit.hpp"
#include "gsr_kspec.hpp"
#include "gsr_interleave16.hpp"
#include "gsr_interleave16d.hpp"
#include "gsr_interleave16c.hpp"

// ---- scratch of the allocation-free entry point ---------------------------------
// gemm_scale_bias_act_noalloc takes the K split's workspace from this array
// instead of an argument: every device the library runs on holds its own
// copy from the time the code object is loaded until the process ends.  It
// is zero-filled at load (uninitialised device data), and the split kernels
// put the arrival counters at its start back to zero at the end of every
// call.  Host code uses the per-device address that hipGetSymbolAddress
// gives, never the array's name, which on the host is only a stand-in.
constexpr int64_t kScratchBytes = (4 << 20) + 512;  // the largest split the library picks: 256 parts of 64x64 fp32 + counters
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

using gsr::Problem;

typedef hipError_t (*launch_fn)(const Problem&, int grid, hipStream_t);

template <typename T>
struct as_is {
    using type = T;
};

// Enqueues `kernel` and returns the status of this launch alone.  The status
// comes from hipLaunchKernel's return value, not from hipGetLastError: an
// error that an earlier, unrelated HIP call left pending on the calling
// thread is neither reported as this launch's nor cleared.
template <typename... P>
hipError_t launch_kernel(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t s, typename as_is<P>::type... args)
{
    void* argv[] = {(void*)&args...};
    return hipLaunchKernel((const void*)kernel, grid, block, argv, 0, s);
}

template <int BM, int BN, int BK, int WM, int WN, bool VEC>
hipError_t launch_staged(const Problem& p, int grid, hipStream_t s)
{
    return launch_kernel((gsr::gemm_scale_relu_kernel<BM, BN, BK, WM, WN, VEC>), dim3(grid),
                         dim3(gsr::kWave * WM * WN), s, p);
}

hipError_t launch_ilv16(const Problem& p, int grid, hipStream_t s)
{
    return launch_kernel(gsr::gemm_scale_relu_ilv16_kernel, dim3(grid), dim3(gsr::Ilv16Cfg::NT), s, p);
}

template <class T>
hipError_t launch_ilv16d(const Problem& p, int grid, hipStream_t s)
{
    return launch_kernel(gsr::gemm_scale_relu_ilv16d_kernel<T>, dim3(grid), dim3(T::NT), s, p);
}

template <class T>
hipError_t launch_ilv16c(const Problem& p, int grid, hipStream_t s)
{
    return launch_kernel(gsr::gemm_scale_relu_ilv16c_kernel<T>, dim3(grid), dim3(T::NT), s, p);
}

template <int BM, int BN, int S>
hipError_t launch_ksplit(const Problem& p, int grid, hipStream_t s)
{
    return launch_kernel((gsr::gemm_scale_relu_ksplit_kernel<BM, BN, S>), dim3(grid), dim3(256), s, p);
}

template <int BM, int BN, int S, int D, bool SPLIT>
hipError_t launch_kspec(const Problem& p, int grid, hipStream_t s)
{
    return launch_kernel((gsr::gemm_scale_relu_kspec_kernel<BM, BN, S, D, SPLIT>), dim3(grid), dim3(512), s, p);
}

struct Entry {
    gsr_config cfg;
    launch_fn vec;       // 128-bit path (16-byte aligned A, B and C, K and N multiples of 8)
    launch_fn elem;      // element-wise path, any 2-byte aligned layout
    int elem_bm, elem_bn;  // the output tile of the element-wise kernel (its grid)
    launch_fn split;     // 128-bit path with K split across workgroups (a workspace), or null
};

// Four waves splitting K inside the workgroup (block_k = 128 per step, waves
// 1 x 1 over the output tile), LDS ring of S stages.  Element-wise path: the
// 64x64 register-staged kernel.
#define GSR_KSPLIT(ID, BM, BN, S, GROUP)                                                              \
    Entry                                                                                             \
    {                                                                                                 \
        {ID, BM, BN, 128, 1, 1, S, GROUP, 1, gsr::KsCfg<BM, BN, S>::LDS_BYTES},                       \
            launch_ksplit<BM, BN, S>, launch_staged<64, 64, 64, 2, 2, false>, 64, 64, nullptr         \
    }

// As GSR_KSPLIT with four more waves that only issue the copies, DEPTH steps
// ahead; with a workspace, the same kernel can also split K across workgroups.
#define GSR_KSPEC(ID, BM, BN, S, D, GROUP)                                                            \
    Entry                                                                                             \
    {                                                                                                 \
        {ID, BM, BN, 128, 1, 1, S, GROUP, 1, gsr::KsCfg<BM, BN, S>::LDS_BYTES},                       \
            launch_kspec<BM, BN, S, D, false>, launch_staged<64, 64, 64, 2, 2, false>, 64, 64,        \
            launch_kspec<BM, BN, S, D, true>                                                          \
    }

// An explicitly interleaved kernel (stages 1: two LDS buffers per operand, or
// two for A and three for B; stages >= 2: a ring of that many A+B buffers);
// its element-wise path is the register-staged kernel of the same tile.
#define GSR_ILV(ID, BM, BN, STAGES, LDS, FN, XCD)                                                          \
    Entry                                                                                                 \
    {                                                                                                     \
        {ID, BM, BN, 64, 2, 2, STAGES, 4, XCD, LDS}, FN, launch_staged<BM, BN, 64, 2, 2, false>, BM, BN,   \
            nullptr                                                                                       \
    }

// The compiled tile table, by id.  Ids are stable from one library version to
// the next, so a tuning table written earlier keeps its meaning; the ids of
// configurations that were dropped (0-15, 19, 20, 23, 24, 26: tiles that
// neither the selector nor any measured tuning entry chose; 15, 23 and 24,
// the 256x256, 128x256 and 128x128 tiles on 32x32x16 MFMAs, were slower than
// configurations 28, 29 and 32 on every measured shape; 26, the 128x256 tile
// with B transposed through registers, is served by 29 and 31; 5, 8 and 10,
// the pipelined 256x128, 128x64 and 64x128 tiles, were the fastest on none of
// the 60 fitting shapes, and the fit without them chooses as well)
// are not reused and are rejected with GSR_ERROR_INVALID_CONFIG.  Tile choice
// per shape class is made by select().
const Entry kTable[] = {
    GSR_KSPLIT(16, 64, 64, 4, 4),            // 4 waves split K, whole 64x64 tile each
    GSR_KSPLIT(17, 64, 32, 6, 4),
    GSR_KSPLIT(18, 32, 64, 6, 4),
    // K split with separate copy waves (eight waves per workgroup), two steps ahead
    GSR_KSPEC(21, 64, 64, 4, 2, 4),
    GSR_KSPEC(22, 32, 64, 4, 2, 4),
    // 256x256 on the 16x16x32 MFMA (8 x 8 blocks of 16x16 per wave), B transposed through
    // registers: configuration 28's twin (same bits), kept for comparison; chip rounds of
    // 16 x 16 tiles where the grid divides into them
    GSR_ILV(25, 256, 256, 1, gsr::Ilv16Cfg::LDS_BYTES, launch_ilv16, 2),
    // configuration 25 with B copied to LDS as stored and read with transpose reads: the
    // selector's 256x256 tile
    GSR_ILV(28, 256, 256, 1, gsr::Ilv16DCfg::LDS_BYTES, launch_ilv16d<gsr::Ilv16DCfg>, 2),
    // configuration 28's kernel on the 128x256 tile (8 x 4 blocks of 16x16 per wave):
    // configuration 31's twin (same bits), kept for comparison
    GSR_ILV(29, 128, 256, 1, gsr::Ilv16HDCfg::LDS_BYTES, launch_ilv16d<gsr::Ilv16HDCfg>, 1),
    // configuration 29 with its copies issued by four extra copy waves (512 threads): the
    // selector's 128x256 tile
    GSR_ILV(31, 128, 256, 1, gsr::Ilv16CCfg::LDS_BYTES, launch_ilv16c<gsr::Ilv16CCfg>, 1),
    // the same kernel on the 128x128 tile (B rows of 256 bytes, 4 x 4 blocks per MFMA wave)
    // with one ring of four A+B stages: the selector's 128x128 tile
    GSR_ILV(32, 128, 128, gsr::Ilv16QCCfg::RING, gsr::Ilv16QCCfg::LDS_BYTES, launch_ilv16c<gsr::Ilv16QCCfg>, 1),
};
constexpr int kNumConfigs = (int)(sizeof(kTable) / sizeof(kTable[0]));

// The table entry of a configuration id, or null for an id that is not compiled.
const Entry* entry_of(int id)
{
    for (const Entry& e : kTable)
        if (e.cfg.id == id) return &e;
    return nullptr;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Tile selection.  A candidate's cost is the time of one tile,
//     2 * bm * bn * K / (per-CU rate) + per-tile overhead,
// times its waves of workgroups on 256 CUs, where a last wave that is not
// full costs max(0.80, 0.35 + 0.65 * fill) of a full one (a part-filled chip
// runs at a higher power-limited clock, but every tile still pays its fixed
// cost).  The 256x256, 128x256 and 128x128 tiles have one candidate each, the
// 16x16x32 kernels with B copied to LDS (configuration 28, and configurations
// 31 and 32 with their copies on separate waves): each was faster than every
// other kernel of its tile on every measured shape.  The
// rates, overheads and the partial-wave form were fitted (least squares in
// relative error for the rates, then the grid point whose choices come
// closest to the fastest configuration) to the times of every configuration
// on 60 shapes measured on one MI355X (M from 1 to 8192 against 11008x4096,
// 4096x4096 and 4096x11008 weights, squares from 256 to 16384, and the
// benchmark workloads), the offline sweep the aikraft.ru guide describes in
// sections 3 and 7 (tiled_dense_gemm_scale_amd/fit_selector.py on
// tuning/mi355x_config_times.csv reproduces this table); on those shapes the
// choice is on average within 0.08 % of the fastest configuration, 2.7 % at
// worst.  Below K = 256 the four-wave K-split tiles replace their copy-wave
// twins (at two K-steps the copy waves have nothing to run ahead of).
struct Candidate {
    int id;
    double tflops_per_cu;  // rate of one CU on this tile while the chip is busy
    double tile_us;        // fixed cost per tile: prologue, epilogue, stores
};
const Candidate kCandidates[] = {
    {28, 6.472, 8.592},   // 256x256, 16x16x32, B copied to LDS
    {31, 6.221, 5.891},   // 128x256, 16x16x32, B copied to LDS by copy waves
    {32, 5.198, 4.377},   // 128x128, 16x16x32, A and B copied to LDS by copy waves
    {21, 2.751, 3.364},   // 64x64, K split, copy waves       (K > 256)
    {22, 1.804, 2.500},   // 32x64, K split, copy waves       (K > 256)
    {16, 2.453, 3.763},   // 64x64, K split, four waves       (K <= 256)
    {18, 1.645, 2.987},   // 32x64, K split, four waves       (K <= 256)
};
constexpr double kPartMin = 0.80, kPartA = 0.35;  // a part-filled last wave: max(kPartMin, kPartA + (1 - kPartA) * fill)

int select(int64_t M, int64_t N, int64_t K)
{
    const double cus = 256.0;
    int best = 28;
    double best_t = 1e300;
    for (const Candidate& c : kCandidates) {
        const bool copy_wave = c.id == 21 || c.id == 22, four_wave = c.id == 16 || c.id == 18;
        if ((copy_wave && K <= 256) || (four_wave && K > 256)) continue;
        const gsr_config& g = entry_of(c.id)->cfg;
        const double wgs = (double)cdiv(M, g.block_m) * (double)cdiv(N, g.block_n);
        const double full = std::floor(wgs / cus), fill = (wgs - full * cus) / cus;
        const double waves = full + (fill > 0.0 ? std::max(kPartMin, kPartA + (1.0 - kPartA) * fill) : 0.0);
        const double tile = 2.0 * g.block_m * g.block_n * (double)(K > 0 ? K : 1) / (c.tflops_per_cu * 1e6) + c.tile_us;
        const double t = waves * tile;
        if (t < best_t) {
            best_t = t;
            best = c.id;
        }
    }
    return best;
}

// ---- K split across workgroups ---------------------------------------------
// The copy-wave K-split tiles (configurations 21 and 22) cover few outputs, so
// shapes with few tiles (decode shapes: a handful of rows against a 4096-wide
// weight) leave most CUs idle while each workgroup streams its whole K range.
// With a workspace the K range of every tile is cut into `parts` runs of
// K-steps, one workgroup each; the parts' fp32 sums meet in the workspace and
// the workgroup of a tile that finishes last adds them (gsr_ksplit.hpp).
// Workspace layout: one 32-bit arrival counter per tile (a region rounded up
// to 256 bytes), then parts x tiles partial tiles of bm x bn fp32, row-major.
constexpr int kSplitStep = 128;    // K-step of the K-split kernels
constexpr int kSplitMaxParts = 16;

struct SplitPlan {
    int parts;       // 1: no split
    int64_t kchunk;  // K values per part (a multiple of kSplitStep)
    int64_t bytes;   // workspace the plan needs
};

int64_t split_count_bytes(int64_t tiles) { return (4 * tiles + 255) / 256 * 256; }

// `want` parts of a tile's K-steps (at most one part per K-step), no part
// empty.
SplitPlan split_plan(int64_t tiles, int bm, int bn, int64_t K, int want)
{
    const int64_t steps = cdiv(K, kSplitStep);
    int64_t parts = std::min<int64_t>(want, steps);
    if (parts <= 1) return SplitPlan{1, K, 0};
    const int64_t per = cdiv(steps, parts);
    parts = cdiv(steps, per);
    if (parts <= 1) return SplitPlan{1, K, 0};
    return SplitPlan{(int)parts, per * kSplitStep,
                     split_count_bytes(tiles) + parts * tiles * (int64_t)bm * bn * 4};
}

// The library's split.  Timed on one MI355X with the 32x64 tile against the
// unsplit kernel (graph replays, 2..16 parts): a part costs about 0.31 us
// per K-step of 128 plus about 1 us per call, and a split adds 2.5-5 us of
// its own (each part's pipeline fill, the partial sums' round trip), so
//  * it pays only from 32 K-steps (K = 4096: 1x4096x4096 11.1 -> 7.8 us,
//    1x2048x4096 9.4 -> 7.2, 8x4096x4096 11.5 -> 8.3; K = 11008:
//    1x4096x11008 28.0 -> 17.7, 16x2048x11008 29.5 -> 13.3; at K = 2048 and
//    1024 it lost 3-30 %);
//  * up to four parts, never more workgroups than CUs (two workgroups of
//    these tiles do not fit one CU: 1024^3 in 512 workgroups took 16 us
//    instead of 6); eight parts were slower than four at 16 and 32 tiles;
//  * with 65-128 tiles, two parts gained where the unsplit call streams well
//    below the part's read ceiling (48x4096x4096 12.9 -> 11.0 us,
//    64x4096x11008 30.7 -> 23.4) and lost 7-10 % where it is near it
//    (1x8192x4096, 16x8192x8192: ~6 TB/s unsplit), so no split when the
//    unsplit call's estimated rate exceeds 4 TB/s.
int split_parts_for(int64_t M, int64_t N, int64_t K, int64_t tiles)
{
    const int64_t steps = cdiv(K, kSplitStep);
    if (steps < 32 || tiles > 128 || tiles <= 0) return 1;
    const double est_us = 1.0 + 0.31 * (double)steps;
    const double bytes = 2.0 * ((double)M * K + (double)K * N + (double)M * N);
    if (bytes / (est_us * 1e-6) > 4e12) return 1;
    return (int)std::max<int64_t>(1, std::min<int64_t>({4, 256 / tiles, steps / 8}));
}

// ---- tuning table: exact shapes -> launch choice ---------------------------
// Written by an offline sweep (tiled_dense_gemm_scale_amd/tune.py) and loaded
// with gsr_load_tuning; a shape found here overrides select().
struct Launch {
    int id, group_m, xcd_remap;
};
struct Tuned {
    int64_t M, N, K;
    Launch l;
};
std::mutex g_tune_mu;
std::vector<Tuned> g_tuned;
std::atomic<bool> g_have_tuning{false};

bool valid_launch(const Launch& l)
{
    return entry_of(l.id) != nullptr && l.group_m >= 1 && l.group_m <= 4096 &&
           l.xcd_remap >= 0 && l.xcd_remap <= 2;
}

// The launch for a problem: a forced config id keeps its compiled launch
// order; otherwise the tuning table, else the selector.
Launch resolve(int64_t M, int64_t N, int64_t K, int config_id)
{
    if (config_id >= 0) return Launch{config_id, entry_of(config_id)->cfg.group_m, entry_of(config_id)->cfg.xcd_remap};
    if (g_have_tuning.load(std::memory_order_acquire)) {
        std::lock_guard<std::mutex> lock(g_tune_mu);
        for (const Tuned& t : g_tuned)
            if (t.M == M && t.N == N && t.K == K) return t.l;
    }
    const int id = select(M, N, K);
    return Launch{id, entry_of(id)->cfg.group_m, entry_of(id)->cfg.xcd_remap};
}

struct DeviceInfo {
    bool ok;
    bool gfx950;
};

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
DeviceInfo g_info[kMaxDevices];

int check_device()
{
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) {
        (void)hipGetLastError();
        return GSR_ERROR_NO_DEVICE;
    }
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return GSR_ERROR_NO_DEVICE;
    }
    std::call_once(g_once[dev], [dev]() {
        hipDeviceProp_t prop;
        DeviceInfo info{false, false};
        if (hipGetDeviceProperties(&prop, dev) == hipSuccess) {
            info.ok = true;
            info.gfx950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        } else {
            (void)hipGetLastError();
        }
        g_info[dev] = info;
    });
    if (!g_info[dev].ok) return GSR_ERROR_NO_DEVICE;
    if (!g_info[dev].gfx950) return GSR_ERROR_UNSUPPORTED_DEVICE;
    return GSR_SUCCESS;
}

// The scratch array's address on the current device, looked up once per
// device (with that device current) on its first use.
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
int g_scratch_status[kMaxDevices];

int scratch_of_current_device(void** out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return GSR_ERROR_NO_DEVICE;
    }
    std::call_once(g_scratch_once[dev], [dev]() {
        void* ptr = nullptr;
        const hipError_t err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (err != hipSuccess || ptr == nullptr) {
            (void)hipGetLastError();
            g_scratch_status[dev] = GSR_ERROR_LAUNCH;
        } else {
            g_scratch_ptr[dev] = ptr;
            g_scratch_status[dev] = GSR_SUCCESS;
        }
    });
    *out = g_scratch_ptr[dev];
    return g_scratch_status[dev];
}

// The element-wise kernel's load unit for an operand whose rows are `len`
// fp16 values long: the largest power of two up to 16 bytes dividing both the
// address and the row length in bytes, so that every row start (and the end
// of the matrix) falls on a multiple of it.
int load_unit(const void* p, int64_t len)
{
    int u = 16;
    while (u > 2 && ((((uintptr_t)p) % (uintptr_t)u) != 0 || ((uint64_t)len * 2u) % (uint64_t)u != 0)) u >>= 1;
    return u;
}

bool overlaps(const void* a, uint64_t abytes, const void* b, uint64_t bbytes)
{
    const uint64_t x = (uint64_t)(uintptr_t)a, y = (uint64_t)(uintptr_t)b;
    return abytes > 0 && bbytes > 0 && x < y + bbytes && y < x + abytes;
}

int validate(int64_t M, int64_t N, int64_t K, const void* A, const void* B, const void* C)
{
    if (M < 0 || N < 0 || K < 0) return GSR_ERROR_INVALID_VALUE;
    const int64_t lim = (int64_t)1 << 31;
    if (M >= lim || N >= lim || K >= lim) return GSR_ERROR_TOO_LARGE;
    if (M == 0 || N == 0) return GSR_SUCCESS;
    if (C == nullptr || ((uintptr_t)C & 1u)) return GSR_ERROR_INVALID_VALUE;
    if (K > 0 && (A == nullptr || B == nullptr || ((uintptr_t)A & 1u) || ((uintptr_t)B & 1u)))
        return GSR_ERROR_INVALID_VALUE;
    // 32-bit byte offsets inside the kernels: every matrix under 2^31 bytes
    const uint64_t abytes = (uint64_t)M * (uint64_t)K * 2u;
    const uint64_t bbytes = (uint64_t)K * (uint64_t)N * 2u;
    const uint64_t cbytes = (uint64_t)M * (uint64_t)N * 2u;
    if (abytes >= (uint64_t)lim || bbytes >= (uint64_t)lim || cbytes >= (uint64_t)lim) return GSR_ERROR_TOO_LARGE;
    if (overlaps(C, cbytes, A, abytes) || overlaps(C, cbytes, B, bbytes)) return GSR_ERROR_INVALID_VALUE;
    return GSR_SUCCESS;
}

}  // namespace

extern "C" {

int gsr_version(void) { return 740; }

const char* gsr_status_string(int status)
{
    switch (status) {
    case GSR_SUCCESS: return "success";
    case GSR_ERROR_INVALID_VALUE: return "invalid value";
    case GSR_ERROR_TOO_LARGE: return "problem too large for 32-bit offsets";
    case GSR_ERROR_NO_DEVICE: return "no HIP device";
    case GSR_ERROR_UNSUPPORTED_DEVICE: return "device is not gfx950";
    case GSR_ERROR_LAUNCH: return "kernel launch failed";
    case GSR_ERROR_INVALID_CONFIG: return "unknown tile configuration";
    default: return "unknown status";
    }
}

int gsr_num_configs(void) { return kNumConfigs; }

int gsr_config_ids(int32_t* ids, int32_t capacity)
{
    if (capacity < 0 || (ids == nullptr && capacity > 0)) return -1;
    for (int i = 0; i < kNumConfigs && i < capacity; ++i) ids[i] = kTable[i].cfg.id;
    return kNumConfigs;
}

int gsr_get_config(int32_t config_id, gsr_config* out)
{
    if (out == nullptr) return GSR_ERROR_INVALID_VALUE;
    const Entry* e = entry_of(config_id);
    if (e == nullptr) return GSR_ERROR_INVALID_CONFIG;
    *out = e->cfg;
    return GSR_SUCCESS;
}

int gsr_select_config(int64_t M, int64_t N, int64_t K, gsr_config* out)
{
    if (out == nullptr || M < 0 || N < 0 || K < 0) return GSR_ERROR_INVALID_VALUE;
    const Launch l = resolve(M, N, K, -1);
    *out = entry_of(l.id)->cfg;
    out->group_m = l.group_m;
    out->xcd_remap = l.xcd_remap;
    return GSR_SUCCESS;
}

}  // extern "C"

namespace {

// Checks, then the launch.  `forced` >= 0 is a config id, -1 the selector,
// -2 the launch in `given`.
// `splits` < 0: no workspace (the entry points without one); 0: the
// library's split when the configuration supports one and the workspace
// holds it (fewer parts until it does); >= 1: that many parts at most, and
// the workspace must hold them.  `use_scratch`: the workspace is this
// device's scratch array, and a split it cannot hold is GSR_ERROR_TOO_LARGE.
int run(int64_t M, int64_t N, int64_t K, const void* A, const void* B, const void* bias, void* C, float alpha,
        int32_t activation, void* stream, int forced, const Launch& given, void* workspace = nullptr,
        int64_t workspace_bytes = 0, int splits = -1, bool use_scratch = false)
{
    int st = validate(M, N, K, A, B, C);
    if (st != GSR_SUCCESS) return st;
    if (!std::isfinite(alpha)) return GSR_ERROR_INVALID_VALUE;
    if (activation != GSR_ACT_RELU && activation != GSR_ACT_GELU && activation != GSR_ACT_NONE)
        return GSR_ERROR_INVALID_VALUE;
    if (bias != nullptr) {
        // read while C is written: it must not overlap C
        if ((uintptr_t)bias & 1u) return GSR_ERROR_INVALID_VALUE;
        if (overlaps(bias, (uint64_t)N * 2u, C, (uint64_t)M * (uint64_t)N * 2u)) return GSR_ERROR_INVALID_VALUE;
    }
    if (forced < -2 || (forced >= 0 && entry_of(forced) == nullptr)) return GSR_ERROR_INVALID_CONFIG;
    if (forced == -2 && !valid_launch(given)) return GSR_ERROR_INVALID_CONFIG;
    if (splits > kSplitMaxParts) return GSR_ERROR_INVALID_VALUE;
    if (splits >= 0 && workspace_bytes < 0) return GSR_ERROR_INVALID_VALUE;
    if (splits >= 0 && workspace != nullptr) {
        // written while A, B and the bias are read and C is written
        if ((uintptr_t)workspace & 15u) return GSR_ERROR_INVALID_VALUE;
        const uint64_t wb = (uint64_t)workspace_bytes;
        if (overlaps(workspace, wb, A, (uint64_t)M * (uint64_t)K * 2u) ||
            overlaps(workspace, wb, B, (uint64_t)K * (uint64_t)N * 2u) ||
            overlaps(workspace, wb, C, (uint64_t)M * (uint64_t)N * 2u) ||
            (bias != nullptr && overlaps(workspace, wb, bias, (uint64_t)N * 2u)))
            return GSR_ERROR_INVALID_VALUE;
    }
    if (M == 0 || N == 0) return GSR_SUCCESS;
    st = check_device();
    if (st != GSR_SUCCESS) return st;
    if (use_scratch) {
        st = scratch_of_current_device(&workspace);
        if (st != GSR_SUCCESS) return st;
        workspace_bytes = kScratchBytes;
    }
    hipStream_t s = (hipStream_t)stream;

    if (K == 0) {
        const uint32_t count = (uint32_t)(M * N);
        const int grid = (int)std::min<int64_t>(cdiv(count, 256), 4096);
        const hipError_t err = launch_kernel(gsr::fill_epilogue_kernel, dim3(grid), dim3(256), s, (uint16_t*)C,
                                             (uint32_t)M, (uint32_t)N, (const uint16_t*)bias, alpha, (int)activation);
        return err == hipSuccess ? GSR_SUCCESS : GSR_ERROR_LAUNCH;
    }

    const Launch l = (forced == -2) ? given : resolve(M, N, K, forced);
    const Entry& e = *entry_of(l.id);
    Problem p;
    p.A = (const uint16_t*)A;
    p.B = (const uint16_t*)B;
    p.C = (uint16_t*)C;
    p.bias = (const uint16_t*)bias;
    p.M = (int)M;
    p.N = (int)N;
    p.K = (int)K;
    p.alpha = alpha;
    p.act = (int)activation;
    // The vector kernels read A and B in 16-byte units and the bias in 8-byte
    // units, and write C in row segments whose starts are 2N bytes apart (a
    // multiple of 16 when N % 8 == 0), in the widest stores C's own alignment
    // allows (p.unit_c); anything else takes the element-wise kernel, whose
    // own tile sets the grid.
    const bool vec = (K % 8 == 0) && (N % 8 == 0) && (((uintptr_t)A & 15u) == 0) &&
                     (((uintptr_t)B & 15u) == 0) && (((uintptr_t)bias & 7u) == 0);
    p.unit_c = load_unit(C, N);
    p.unit_a = load_unit(A, K);
    p.unit_b = load_unit(B, N);
    p.tiles_m = (int)cdiv(M, vec ? e.cfg.block_m : e.elem_bm);
    p.tiles_n = (int)cdiv(N, vec ? e.cfg.block_n : e.elem_bn);
    p.group_m = l.group_m;
    p.xcd_remap = l.xcd_remap;
    p.ksplit = 1;
    p.kchunk = (int)K;
    p.ws_part = nullptr;
    p.ws_count = nullptr;
    const int tiles = p.tiles_m * p.tiles_n;
    SplitPlan plan{1, K, 0};
    if (splits > 1 && !(vec && e.split != nullptr)) {
        // a forced split that this configuration or layout cannot run
        if (e.split == nullptr) return GSR_ERROR_INVALID_CONFIG;
    } else if (splits >= 0 && vec && e.split != nullptr) {
        const int want = splits > 0 ? splits : split_parts_for(M, N, K, tiles);
        plan = split_plan(tiles, e.cfg.block_m, e.cfg.block_n, K, want);
        if (plan.parts > 1 && (workspace == nullptr || workspace_bytes < plan.bytes)) {
            if (use_scratch) return GSR_ERROR_TOO_LARGE;      // beyond the scratch array
            if (splits > 0) return GSR_ERROR_INVALID_VALUE;  // the workspace cannot hold the forced split
            while (plan.parts > 1 && (workspace == nullptr || workspace_bytes < plan.bytes))
                plan = split_plan(tiles, e.cfg.block_m, e.cfg.block_n, K, plan.parts - 1);
        }
    }
    if (plan.parts > 1) {
        p.ksplit = plan.parts;
        p.kchunk = (int)plan.kchunk;
        p.ws_count = (uint32_t*)workspace;
        p.ws_part = (float*)((uint8_t*)workspace + split_count_bytes(tiles));
        const hipError_t err = e.split(p, tiles * plan.parts, s);
        return err == hipSuccess ? GSR_SUCCESS : GSR_ERROR_LAUNCH;
    }
    const hipError_t err = (vec ? e.vec : e.elem)(p, tiles, s);
    return err == hipSuccess ? GSR_SUCCESS : GSR_ERROR_LAUNCH;
}

}  // namespace

extern "C" {

int gemm_scale_bias_act_ex(int64_t M, int64_t N, int64_t K, const void* A, const void* B, const void* bias,
                           void* C, float alpha, int32_t activation, void* stream, int32_t config_id)
{
    if (config_id < -1) return GSR_ERROR_INVALID_CONFIG;
    return run(M, N, K, A, B, bias, C, alpha, activation, stream, config_id, Launch{0, 0, 0});
}

int gemm_scale_bias_act_cfg(int64_t M, int64_t N, int64_t K, const void* A, const void* B, const void* bias,
                            void* C, float alpha, int32_t activation, void* stream, const gsr_config* cfg)
{
    if (cfg == nullptr) return GSR_ERROR_INVALID_VALUE;
    return run(M, N, K, A, B, bias, C, alpha, activation, stream, -2, Launch{cfg->id, cfg->group_m, cfg->xcd_remap});
}

int gsr_load_tuning(const char* path)
{
    if (path == nullptr) return GSR_ERROR_INVALID_VALUE;
    FILE* f = std::fopen(path, "r");
    if (f == nullptr) return GSR_ERROR_INVALID_VALUE;
    std::vector<Tuned> table;
    char line[512];
    int st = GSR_SUCCESS;
    while (std::fgets(line, sizeof line, f) != nullptr) {
        char* hash = std::strchr(line, '#');
        if (hash != nullptr) *hash = 0;
        long long m, n, k;
        int id, gm, xr;
        char extra;
        const int got = std::sscanf(line, "%lld %lld %lld %d %d %d %c", &m, &n, &k, &id, &gm, &xr, &extra);
        if (got <= 0) {  // blank or comment line
            bool blank = true;
            for (const char* c = line; *c; ++c)
                if (*c != ' ' && *c != '\t' && *c != '\n' && *c != '\r') blank = false;
            if (blank) continue;
            st = GSR_ERROR_INVALID_VALUE;
            break;
        }
        const Tuned t{m, n, k, Launch{id, gm, xr}};
        if (got != 6 || m < 0 || n < 0 || k < 0 || !valid_launch(t.l)) {
            st = GSR_ERROR_INVALID_VALUE;
            break;
        }
        table.push_back(t);
    }
    std::fclose(f);
    if (st != GSR_SUCCESS) return st;  // the previous table stays
    std::lock_guard<std::mutex> lock(g_tune_mu);
    g_tuned.swap(table);
    g_have_tuning.store(!g_tuned.empty(), std::memory_order_release);
    return GSR_SUCCESS;
}

int gsr_clear_tuning(void)
{
    std::lock_guard<std::mutex> lock(g_tune_mu);
    g_tuned.clear();
    g_have_tuning.store(false, std::memory_order_release);
    return GSR_SUCCESS;
}

int gsr_tuning_entries(void)
{
    std::lock_guard<std::mutex> lock(g_tune_mu);
    return (int)g_tuned.size();
}

int gemm_scale_bias_act(int64_t M, int64_t N, int64_t K, const void* A, const void* B, const void* bias,
                        void* C, float alpha, int32_t activation, void* stream)
{
    return gemm_scale_bias_act_ex(M, N, K, A, B, bias, C, alpha, activation, stream, -1);
}

int gemm_scale_relu_ex(int64_t M, int64_t N, int64_t K, const void* A, const void* B, void* C, float alpha,
                       void* stream, int32_t config_id)
{
    return gemm_scale_bias_act_ex(M, N, K, A, B, nullptr, C, alpha, GSR_ACT_RELU, stream, config_id);
}

int gemm_scale_relu(int64_t M, int64_t N, int64_t K, const void* A, const void* B, void* C, float alpha,
                    void* stream)
{
    return gemm_scale_bias_act_ex(M, N, K, A, B, nullptr, C, alpha, GSR_ACT_RELU, stream, -1);
}

int gemm_scale_bias_act_ws(int64_t M, int64_t N, int64_t K, const void* A, const void* B, const void* bias,
                           void* C, float alpha, int32_t activation, void* workspace, int64_t workspace_bytes,
                           void* stream, int32_t config_id, int32_t splits)
{
    if (config_id < -1) return GSR_ERROR_INVALID_CONFIG;
    if (splits < 0) return GSR_ERROR_INVALID_VALUE;
    return run(M, N, K, A, B, bias, C, alpha, activation, stream, config_id, Launch{0, 0, 0}, workspace,
               workspace_bytes, splits);
}

int gemm_scale_relu_ws(int64_t M, int64_t N, int64_t K, const void* A, const void* B, void* C, float alpha,
                       void* workspace, int64_t workspace_bytes, void* stream)
{
    return gemm_scale_bias_act_ws(M, N, K, A, B, nullptr, C, alpha, GSR_ACT_RELU, workspace, workspace_bytes,
                                  stream, -1, 0);
}

int gemm_scale_bias_act_noalloc(int64_t M, int64_t N, int64_t K, const void* A, const void* B, const void* bias,
                                void* C, float alpha, int32_t activation, void* stream, int32_t config_id,
                                int32_t splits)
{
    if (config_id < -1) return GSR_ERROR_INVALID_CONFIG;
    if (splits < 0) return GSR_ERROR_INVALID_VALUE;
    return run(M, N, K, A, B, bias, C, alpha, activation, stream, config_id, Launch{0, 0, 0}, nullptr, 0, splits,
               true);
}

int64_t gsr_workspace_bytes(int64_t M, int64_t N, int64_t K)
{
    if (M < 0 || N < 0 || K < 0) return -1;
    if (M == 0 || N == 0 || K == 0) return 0;
    const Launch l = resolve(M, N, K, -1);
    const Entry& e = *entry_of(l.id);
    if (e.split == nullptr) return 0;
    const int64_t tiles = cdiv(M, e.cfg.block_m) * cdiv(N, e.cfg.block_n);
    return split_plan(tiles, e.cfg.block_m, e.cfg.block_n, K, split_parts_for(M, N, K, tiles)).bytes;
}

}  // extern "C"
