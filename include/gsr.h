/*
 * gsr.h -- C ABI of the fused fp16 GEMM + scale + ReLU library for AMD
 * Instinct MI355X (gfx950).
 *
 * The operation (PKUHPC scow-tutorial "Tutorial14: 使用TileLang语言编写attention
 * 算子", section 3 "算子介绍", display formula and symbol list; the kernel
 * listing in section 2 "编写算子" fixes the types and the epilogue order):
 *
 *     C[m,n] = ReLU( alpha * sum_{k<K} A[m,k] * B[k,n] ),  ReLU(x) = max(x, 0)
 *
 *   A  M x K, IEEE binary16, row-major (leading dimension K)
 *   B  K x N, IEEE binary16, row-major (leading dimension N)
 *   C  M x N, IEEE binary16, row-major (leading dimension N), written once
 *   alpha  binary32 scalar
 * Products are accumulated in binary32; the scale and the max(., 0) are applied
 * to the binary32 sum in registers and the result is narrowed to binary16 with
 * round-to-nearest-even on the single store.  Non-positive results are +0.
 *
 * Ownership and ordering.  A, B and C are device pointers owned by the caller
 * (any allocation the HIP runtime can address from the current device).  The
 * library allocates nothing and keeps no per-call state (the entry points
 * with a workspace keep theirs in the caller's workspace); it only enqueues
 * kernels on `stream` (a hipStream_t; NULL means the null stream) and returns
 * before they finish.  The caller synchronises.  Calls are thread-safe.
 *
 * Error behaviour.  Arguments are checked on the host before anything is
 * enqueued; a nonzero status means nothing was launched (except
 * GSR_ERROR_LAUNCH, which reports a failed launch).  No status aborts the
 * process.
 */
#ifndef GSR_H_
#define GSR_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum gsr_status {
    GSR_SUCCESS = 0,
    /* a dimension < 0; a null or odd-address pointer where the extent is
     * nonzero; C's byte range overlapping A's or B's; alpha not finite */
    GSR_ERROR_INVALID_VALUE = 1,
    /* a dimension >= 2^31, or a matrix of 2^31 bytes or more (the kernels
     * use 32-bit byte offsets) */
    GSR_ERROR_TOO_LARGE = 2,
    GSR_ERROR_NO_DEVICE = 3,          /* no HIP device is visible */
    GSR_ERROR_UNSUPPORTED_DEVICE = 4, /* the current device is not gfx950 */
    GSR_ERROR_LAUNCH = 5,             /* the runtime rejected the launch */
    GSR_ERROR_INVALID_CONFIG = 6      /* gemm_scale_relu_ex: unknown config id */
};

/* Activation of the epilogue variants. */
enum gsr_activation {
    GSR_ACT_RELU = 0, /* max(v, 0); non-positive results are +0 */
    GSR_ACT_GELU = 1, /* v/2 * (1 + tanh(sqrt(2/pi) * (v + 0.044715 v^3))) */
    GSR_ACT_NONE = 2  /* v itself */
};

/* One compiled tile configuration.  A workgroup of waves_m*waves_n wave64s
 * owns a block_m x block_n tile of C and walks K in steps of block_k through
 * `stages` LDS buffers (0 or 1: two per operand; configurations 28, 29 and
 * 31: two for A, three for B; 2 or more: a ring of that many buffers per
 * operand); each wave owns a (block_m/waves_m) x (block_n/waves_n) sub-tile
 * (configurations 31 and 32 add waves_m * waves_n waves that only copy
 * operands into LDS).  Configurations 25, 28, 29, 31 and 32 build that
 * sub-tile from 16x16x32 fp16 MFMAs, all others from 32x32x16 fp16 MFMAs.  (The K-split kinds, block_k
 * 128 with waves 1 x 1, give every wave the whole tile and a share of each
 * K-step instead.)  group_m is the number of tile rows in one group of the
 * grouped launch order; xcd_remap picks how workgroup ids map to tiles: 0 the
 * grouped order on the ids as dispatched, 1 the same on ids regrouped so that
 * neighbouring tiles run on the same XCD, 2 chip-wide rounds of 16 x 16 tiles
 * with a 4 x 8 part per XCD (grids whose tile rows and columns are multiples
 * of 16; others use 1; group_m unused).  Ids are stable across library
 * versions and not contiguous: gsr_config_ids lists the compiled ones. */
typedef struct gsr_config {
    int32_t id;
    int32_t block_m, block_n, block_k;
    int32_t waves_m, waves_n;
    int32_t stages;
    int32_t group_m;
    int32_t xcd_remap;
    int32_t lds_bytes;
} gsr_config;

/* The fused operation (the tutorial's kernel call: A, B, C, scale).
 * M, N, K >= 0.  M == 0 or N == 0: success, nothing enqueued.  K == 0: every
 * output is the empty sum, C is filled with +0.  Any pointer alignment of at
 * least 2 bytes is accepted; 16-byte aligned A and B with K and N multiples
 * of 8 take the 128-bit vector path (C written in the widest stores its own
 * alignment allows), anything else an element-wise path (a register-staged
 * kernel of the same tile, or of a 64x64 tile for the K-split kinds, reading
 * each operand in the widest unit its alignment allows).  Returns a gsr_status. */
int gemm_scale_relu(int64_t M, int64_t N, int64_t K,
                    const void* A, const void* B, void* C,
                    float alpha, void* stream);

/* As gemm_scale_relu with a forced tile configuration (an id from
 * gsr_config_ids; -1 = the selector's choice).  For sweeps and tests. */
int gemm_scale_relu_ex(int64_t M, int64_t N, int64_t K,
                       const void* A, const void* B, void* C,
                       float alpha, void* stream, int32_t config_id);

/* The epilogue variants (the aikraft.ru TileLang guide, section 4 "Слияние
 * эпилогов: GEMM + Bias + GELU": a bias and an exponent-based GELU applied to
 * the matmul result in registers before the single store):
 *
 *     C[m,n] = act( alpha * sum_{k<K} A[m,k] * B[k,n] + bias[n] )
 *
 *   bias  NULL, or N IEEE binary16 values on the device (one per output
 *         column, at least 2-byte aligned; 8-byte alignment keeps the 128-bit
 *         path), read-only, must not overlap C
 *   activation  a gsr_activation; GELU is the tanh form, evaluated in binary32
 *         as v / (1 + exp(-2u)), u = sqrt(2/pi) (v + 0.044715 v^3)
 * The sum, the scale, the bias and the activation are binary32; one
 * round-to-nearest-even narrowing to binary16.  With bias == NULL and
 * GSR_ACT_RELU this is exactly gemm_scale_relu; the guide's GEMM + Bias + GELU
 * is alpha = 1, GSR_ACT_GELU.  K == 0 gives act(bias[n]) (+0 without a bias).
 * Layout, alignment, ownership and errors as gemm_scale_relu; in addition
 * GSR_ERROR_INVALID_VALUE for an unknown activation, an odd bias address or
 * a bias overlapping C. */
int gemm_scale_bias_act(int64_t M, int64_t N, int64_t K,
                        const void* A, const void* B, const void* bias, void* C,
                        float alpha, int32_t activation, void* stream);

/* As gemm_scale_bias_act with a forced tile configuration (-1 = selector). */
int gemm_scale_bias_act_ex(int64_t M, int64_t N, int64_t K,
                           const void* A, const void* B, const void* bias, void* C,
                           float alpha, int32_t activation, void* stream, int32_t config_id);

/* As gemm_scale_bias_act with an explicit launch: cfg->id picks the compiled
 * tile configuration; cfg->group_m (1..4096, tile rows per group of the
 * launch order) and cfg->xcd_remap (0, 1 or 2) override that configuration's
 * launch order; the other fields are ignored.  The launch order changes only
 * which tiles run together, never a tile's arithmetic, so results are bit
 * for bit those of gemm_scale_bias_act_ex with the same id.  For tuning
 * sweeps.  GSR_ERROR_INVALID_CONFIG for an out-of-range field. */
int gemm_scale_bias_act_cfg(int64_t M, int64_t N, int64_t K,
                            const void* A, const void* B, const void* bias, void* C,
                            float alpha, int32_t activation, void* stream, const gsr_config* cfg);

/* The same operations with a workspace, so that K can be split across
 * workgroups.  The pages do not describe splitting K: the sum is still the
 * one the PKUHPC tutorial defines (section 3 display formula), taken over
 * runs of K and added, and the context is the aikraft.ru guide's section 3
 * (no schedule is best for every size) and the TileKernels article's section
 * one (memory bandwidth utilisation as the measure of a memory-bound
 * product).  It serves shapes whose output has too few tiles of the K-split
 * kinds (configurations 21 and 22) to occupy the chip, such as a few rows
 * against a 4096-wide weight: each tile's
 * K-steps are cut into `parts` runs, one workgroup each, whose fp32 sums meet
 * in the workspace, and the workgroup of a tile that finishes last adds them
 * in part order, applies the epilogue and stores C.  The sum of a part is
 * that of the unsplit kernel over its K range, so results differ from the
 * unsplit call only by the order of fp32 additions.
 *
 *   workspace  device memory owned by the caller, 16-byte aligned, not
 *              overlapping A, B, C or the bias.  Its first bytes hold one
 *              32-bit arrival counter per tile and must be zero before the
 *              first call (allocate it zero-filled); every call leaves them
 *              zero again, so the same workspace serves any number of calls
 *              in stream order.  Calls that may run at the same time (other
 *              streams, other threads) need workspaces of their own.
 *   workspace_bytes  its size; gsr_workspace_bytes gives what the library's
 *              choice needs (at most 4 MiB + 512 bytes for any shape)
 *   splits     0: the library's choice (shapes of at most 128 such tiles
 *              and at least 32 K-steps of 128 whose unsplit call would not
 *              already stream near the read ceiling: up to four parts, at
 *              most one workgroup per CU and eight K-steps per part; fewer
 *              parts when the workspace is smaller, none without one);
 *              n >= 1: at most n parts (never
 *              more than one per K-step), GSR_ERROR_INVALID_VALUE if the
 *              workspace cannot hold them, GSR_ERROR_INVALID_CONFIG for n > 1
 *              with a configuration that cannot split.  1..16.
 * A call that does not split (other configurations, the element-wise path,
 * parts = 1) ignores the workspace.  Otherwise as gemm_scale_bias_act_ex and
 * gemm_scale_relu; GSR_ERROR_INVALID_VALUE also for a misaligned or
 * overlapping workspace, a negative size or splits outside 0..16. */
int gemm_scale_bias_act_ws(int64_t M, int64_t N, int64_t K,
                           const void* A, const void* B, const void* bias, void* C,
                           float alpha, int32_t activation,
                           void* workspace, int64_t workspace_bytes,
                           void* stream, int32_t config_id, int32_t splits);

/* gemm_scale_relu with a workspace: the selector's configuration and the
 * library's split. */
int gemm_scale_relu_ws(int64_t M, int64_t N, int64_t K,
                       const void* A, const void* B, void* C, float alpha,
                       void* workspace, int64_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * gemm_scale_bias_act_ws with the workspace taken from a scratch array that
 * the library keeps in every device's memory (4 MiB + 512 bytes per device,
 * present from the time the library's code object is loaded until the
 * process ends; its address is looked up once per device, on the first call
 * with that device current, so under graph capture make one call outside
 * the capture first).  The call itself allocates nothing.  Every call
 * on one device shares that device's array: calls that may overlap on one
 * device (other streams, other threads, other libraries' copies excepted)
 * race, and their results and the array's arrival counters are then
 * undefined.  Calls in stream order are safe: the counters start at zero and
 * every call leaves them zero.  A split that needs more than the array holds
 * (only a forced `splits` can) is GSR_ERROR_TOO_LARGE, with nothing
 * enqueued; the library's own choice always fits.  GSR_ERROR_LAUNCH also
 * when the runtime cannot give the array's address.  Otherwise as
 * gemm_scale_bias_act_ws. */
int gemm_scale_bias_act_noalloc(int64_t M, int64_t N, int64_t K,
                                const void* A, const void* B, const void* bias, void* C,
                                float alpha, int32_t activation,
                                void* stream, int32_t config_id, int32_t splits);

/* Workspace bytes the library's split needs for an M x N x K call on the
 * 128-bit path (the selector's or the tuning table's configuration); 0 when
 * that call does not split, -1 for a negative dimension.  Host only. */
int64_t gsr_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* Tuning table: exact problem shapes mapped to a launch, consulted before the
 * built-in selector (by every entry point called with config id -1, and by
 * gsr_select_config).  The file is text, one entry per line,
 *     M N K config_id group_m xcd_remap
 * with '#' starting a comment; tiled_dense_gemm_scale_amd/tune.py writes it
 * from measured sweeps (the aikraft.ru TileLang guide: section 3, a manual
 * sweep of tile, stage and swizzle knobs that finds no schedule best for
 * every size; section 7, an automatic search of that space per problem and
 * GPU).  gsr_load_tuning replaces the table, or returns
 * GSR_ERROR_INVALID_VALUE for an unreadable or malformed file and keeps the
 * previous one; gsr_clear_tuning empties it; gsr_tuning_entries counts it.
 * Host only, thread-safe. */
int gsr_load_tuning(const char* path);
int gsr_clear_tuning(void);
int gsr_tuning_entries(void);

/* The configuration the selector picks for an M x N x K problem (the tuning
 * table first, with its launch order in group_m / xcd_remap).  Host only;
 * touches no device.  Returns GSR_SUCCESS or GSR_ERROR_INVALID_VALUE. */
int gsr_select_config(int64_t M, int64_t N, int64_t K, gsr_config* out);

/* Number of compiled tile configurations; their ids (written to ids[0..],
 * at most `capacity` of them; returns the number of compiled configurations,
 * or -1 for capacity < 0 or a null ids with capacity > 0); the description of
 * one (GSR_ERROR_INVALID_CONFIG for an id that is not compiled).  Host only. */
int gsr_num_configs(void);
int gsr_config_ids(int32_t* ids, int32_t capacity);
int gsr_get_config(int32_t config_id, gsr_config* out);

/* A static, human-readable name for a status code. */
const char* gsr_status_string(int status);

/* Library version, as major*10000 + minor*100 + patch. */
int gsr_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GSR_H_ */
