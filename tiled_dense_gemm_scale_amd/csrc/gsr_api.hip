// gsr_api.hip -- host side of the C ABI declared in include/gsr.h: argument
// checks, device check, tile selection and the launch on the caller's stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "gsr.h"
#include "gsr_kernels.hpp"

namespace {

using gsr::Problem;

typedef hipError_t (*launch_fn)(const Problem&, int grid, hipStream_t);

template <int BM, int BN, int BK, int WM, int WN, bool VEC>
hipError_t launch(const Problem& p, int grid, hipStream_t s)
{
    hipLaunchKernelGGL((gsr::gemm_scale_relu_kernel<BM, BN, BK, WM, WN, VEC>), dim3(grid),
                       dim3(gsr::kWave * WM * WN), 0, s, p);
    return hipGetLastError();
}

struct Entry {
    gsr_config cfg;
    launch_fn vec;   // 128-bit path
    launch_fn elem;  // element-wise path
};

#define GSR_ENTRY(ID, BM, BN, BK, WM, WN, GROUP)                                                      \
    Entry                                                                                             \
    {                                                                                                 \
        {ID, BM, BN, BK, WM, WN, 2, GROUP, 1, gsr::TileKernel<BM, BN, BK, WM, WN, true>::LDS_BYTES}, \
            launch<BM, BN, BK, WM, WN, true>, launch<BM, BN, BK, WM, WN, false>                      \
    }

// The compiled tile table.  Tile choice per shape class is made by select().
const Entry kTable[] = {
    GSR_ENTRY(0, 256, 256, 64, 2, 4, 4),  // large: 8 waves of 128x64
    GSR_ENTRY(1, 256, 128, 64, 2, 2, 4),  // 4 waves of 128x64
    GSR_ENTRY(2, 128, 256, 64, 2, 2, 4),  // 4 waves of 64x128
    GSR_ENTRY(3, 128, 128, 64, 2, 2, 4),  // 4 waves of 64x64
    GSR_ENTRY(4, 128, 64, 64, 2, 2, 4),   // 4 waves of 64x32
    GSR_ENTRY(5, 64, 64, 64, 2, 2, 4),    // small: 4 waves of 32x32
};
constexpr int kNumConfigs = (int)(sizeof(kTable) / sizeof(kTable[0]));

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Shape classes: enough workgroups to cover the 256 CUs with the largest
// tile that still does so; otherwise fall back to smaller tiles.
int select(int64_t M, int64_t N, int64_t /*K*/)
{
    const int64_t cus = 256;
    const int order[] = {0, 1, 2, 3, 4, 5};
    for (int id : order) {
        const gsr_config& c = kTable[id].cfg;
        const int64_t wgs = cdiv(M, c.block_m) * cdiv(N, c.block_n);
        if (wgs >= cus) return id;
    }
    return 5;
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

int gsr_version(void) { return 100; }

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

int gsr_get_config(int32_t config_id, gsr_config* out)
{
    if (out == nullptr) return GSR_ERROR_INVALID_VALUE;
    if (config_id < 0 || config_id >= kNumConfigs) return GSR_ERROR_INVALID_CONFIG;
    *out = kTable[config_id].cfg;
    return GSR_SUCCESS;
}

int gsr_select_config(int64_t M, int64_t N, int64_t K, gsr_config* out)
{
    if (out == nullptr || M < 0 || N < 0 || K < 0) return GSR_ERROR_INVALID_VALUE;
    *out = kTable[select(M, N, K)].cfg;
    return GSR_SUCCESS;
}

int gemm_scale_relu_ex(int64_t M, int64_t N, int64_t K, const void* A, const void* B, void* C, float alpha,
                       void* stream, int32_t config_id)
{
    int st = validate(M, N, K, A, B, C);
    if (st != GSR_SUCCESS) return st;
    if (!std::isfinite(alpha)) return GSR_ERROR_INVALID_VALUE;
    if (config_id < -1 || config_id >= kNumConfigs) return GSR_ERROR_INVALID_CONFIG;
    if (M == 0 || N == 0) return GSR_SUCCESS;
    st = check_device();
    if (st != GSR_SUCCESS) return st;
    hipStream_t s = (hipStream_t)stream;

    if (K == 0) {
        const uint32_t count = (uint32_t)(M * N);
        const int grid = (int)std::min<int64_t>(cdiv(count, 256), 4096);
        hipLaunchKernelGGL(gsr::fill_zero_kernel, dim3(grid), dim3(256), 0, s, (uint16_t*)C, count);
        return hipGetLastError() == hipSuccess ? GSR_SUCCESS : GSR_ERROR_LAUNCH;
    }

    const Entry& e = kTable[config_id < 0 ? select(M, N, K) : config_id];
    Problem p;
    p.A = (const uint16_t*)A;
    p.B = (const uint16_t*)B;
    p.C = (uint16_t*)C;
    p.M = (int)M;
    p.N = (int)N;
    p.K = (int)K;
    p.alpha = alpha;
    p.tiles_m = (int)cdiv(M, e.cfg.block_m);
    p.tiles_n = (int)cdiv(N, e.cfg.block_n);
    p.group_m = e.cfg.group_m;
    p.xcd_remap = e.cfg.xcd_remap;
    const int grid = p.tiles_m * p.tiles_n;
    const bool vec = (K % 8 == 0) && (N % 8 == 0) && (((uintptr_t)A & 15u) == 0) &&
                     (((uintptr_t)B & 15u) == 0) && (((uintptr_t)C & 7u) == 0);
    const hipError_t err = (vec ? e.vec : e.elem)(p, grid, s);
    return err == hipSuccess ? GSR_SUCCESS : GSR_ERROR_LAUNCH;
}

int gemm_scale_relu(int64_t M, int64_t N, int64_t K, const void* A, const void* B, void* C, float alpha,
                    void* stream)
{
    return gemm_scale_relu_ex(M, N, K, A, B, C, alpha, stream, -1);
}

}  // extern "C"
