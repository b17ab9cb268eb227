/*
 * fused_ar.h - C ABI of libfused_ar.so: the fused all-reduce + residual-add + RMSNorm epilogue
 * on one MI355X (gfx950), for the N partial sums that N tensor-parallel ranks would hold.
 *
 * What it computes (one GPU's share of the fused operator):
 *   reduced[r][j]      = bf16( fp32 sum of inputs[0][r][j], ..., inputs[n-1][r][j], left to right )
 *   residual_out[r][j] = bf16( reduced[r][j] + residual[r][j] )
 *   out[r][j]          = bf16( residual_out[r][j] / sqrt(mean_j(residual_out[r][j]^2) + eps) * weight[j] )
 * - the reduce: "perf: optimize fused AllReduce + RMSNorm (custom_all_reduce)" (ROCm/aiter
 *   PR #3817), Technical Details > 2stage > reduce-scatter (per-pack fp32 reduce across the ranks
 *   in the order ptrs[0..ngpus-1], then a downcast to bf16);
 * - residual add and RMSNorm: the fused operator of "perf(comm): add opt-in Triton AR+RMSNorm
 *   backend" (lightseekorg/tokenspeed PR #968), Summary (AI), on contiguous bf16 (tokens, hidden)
 *   tensors with a bf16 weight; the RMSNorm square-sum is a per-row reduction (aiter PR #3817,
 *   Technical Details > 1stage and > 2stage > stage-2 RMSNorm reduce).
 * Conversions to bf16 round to nearest, ties to even. The sums of the reduce are exact binary32
 * additions in the fixed order, so `reduced` and `residual_out` are reproducible bit for bit; the
 * RMSNorm statistic is an fp32 sum in a fixed tree, so `out` is deterministic run to run.
 *
 * Conventions for every entry point:
 * - bf16 values are raw 16-bit patterns (fa_bf16). Every [m, hidden] array is row-major and
 *   contiguous, so row r starts hidden elements after row r-1; `weight` has hidden elements.
 * - Pointers named "device" are device (HBM) addresses on the current HIP device; the caller owns
 *   all of them. The library allocates nothing, keeps no state between calls (apart from the fixed
 *   scratch of fused_ar_rmsnorm_split_static, below) and never synchronises: it enqueues kernels
 *   on `stream` and returns. Buffers must stay valid until the
 *   stream has executed the work. Calls may be captured into a HIP graph (the pointers are copied
 *   into the kernel arguments and are baked into the graph).
 * - `inputs` is a HOST array of n device pointers; it is read during the call only.
 * - Every argument check happens before any HIP call. A rejected call launches nothing.
 * - Return value: FUSED_AR_OK (0), one of the negative FUSED_AR_ERR_* codes below, or a positive
 *   hipError_t reported by the kernel launch. fused_ar_strerror() names each.
 */
#ifndef FUSED_AR_H
#define FUSED_AR_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t fa_bf16; /* raw bfloat16 bit pattern */

enum {
    FUSED_AR_OK = 0,
    FUSED_AR_ERR_INVALID = -1, /* null pointer, n outside [1, 8], m < 0, hidden <= 0, eps < 0 or
                                  not finite, path outside {0, 1, 2}, pointer range wraps */
    FUSED_AR_ERR_SHAPE = -2,   /* hidden not a multiple of 8, or above FUSED_AR_MAX_HIDDEN; or a
                                  row (slice) that does not fit 1024 threads at the packs per
                                  thread (slices) a caller forced */
    FUSED_AR_ERR_ALIGN = -3,   /* a device pointer not 16-byte aligned */
    FUSED_AR_ERR_ALIAS = -4,   /* a forbidden overlap of buffers (see fused_ar_rmsnorm) */
    FUSED_AR_ERR_SCRATCH = -5  /* fused_ar_rmsnorm_split_static: m * slices above
                                  FUSED_AR_STATIC_SCRATCH_FLOATS */
};

#define FUSED_AR_MAX_INPUTS 8
#define FUSED_AR_MAX_HIDDEN 32768

/* Path selector values. */
enum {
    FUSED_AR_PATH_AUTO = 0,     /* fused_ar_auto_path(n, m, hidden) */
    FUSED_AR_PATH_ONESTAGE = 1, /* one kernel, one row per workgroup */
    FUSED_AR_PATH_TWOSTAGE = 2, /* a flat reduce kernel (by default it also adds the residual),
                                   then an RMSNorm kernel; see FUSED_AR_RESIDUAL_* */
    FUSED_AR_PATH_UNFUSED = 3   /* reduce, residual add and RMSNorm as three kernels (only through
                                   fused_ar_unfused_rmsnorm, fused_ar_rmsnorm_ex and
                                   fused_ar_describe_launch) */
};

/*
 * fused_ar_rmsnorm - the whole epilogue: reduce, residual add, RMSNorm.
 *
 *   inputs        host array of n device pointers, each [m, hidden] bf16; the reduce order is the
 *                 array order (aiter PR #3817, Technical Details > 2stage > reduce-scatter).
 *   n             number of partial sums, 1..FUSED_AR_MAX_INPUTS.
 *   residual      device [m, hidden] bf16.
 *   weight        device [hidden] bf16.
 *   eps           >= 0 and finite; added to the mean of squares inside the square root. With
 *                 eps == 0 a row that is all zero gives NaN (0 * inf), as the formula does. With
 *                 eps below 2^-126 (0 or subnormal), rows so small that their fp32 square-sum is
 *                 below 2^-110 are summed again at a 2^100 scale, so that squares in or under
 *                 fp32's subnormal range keep their bits. The statistic is fp32: rows whose
 *                 square-sum exceeds fp32's range (|x| above about 1.8e19) give out = 0.
 *   m, hidden     rows (tokens) and row length; m == 0 returns FUSED_AR_OK and launches nothing
 *                 (no pointer is looked at); hidden % 8 == 0 and hidden <= FUSED_AR_MAX_HIDDEN.
 *   residual_out  device [m, hidden] bf16, written. May be exactly `residual` (in place); it must
 *                 not otherwise overlap `residual`, and must not overlap an input or the weight.
 *   out           device [m, hidden] bf16, written. Must not overlap any other buffer. The
 *                 two-stage path in the pages' split (see FUSED_AR_RESIDUAL_STAGE2) also uses it
 *                 as its scratch: stage 1 writes the reduced rows there and stage 2 overwrites
 *                 them with the normalised rows.
 *   path          FUSED_AR_PATH_AUTO, _ONESTAGE or _TWOSTAGE (aiter PR #3817, Technical Details >
 *                 1stage / 2stage); both give bit-identical residual_out and out (the row kernels
 *                 of a call share one geometry and one reduction tree).
 *   stream        HIP stream the kernels are enqueued on (0 = the null stream).
 * Inputs may overlap one another and the weight may overlap inputs or the residual (all are only
 * read). All device pointers must be 16-byte aligned.
 */
int fused_ar_rmsnorm(const fa_bf16 *const *inputs, int n, const fa_bf16 *residual,
                     const fa_bf16 *weight, float eps, int m, int hidden, fa_bf16 *residual_out,
                     fa_bf16 *out, int path, hipStream_t stream);

/*
 * fused_ar_unfused_rmsnorm - the same result as fused_ar_rmsnorm, bit for bit, computed the way an
 * unfused epilogue would: an all-reduce (the flat reduce kernel) writing the reduced rows to
 * `out`, a residual add writing residual_out, then an RMSNorm kernel reading residual_out back and
 * writing out. The baseline that the fused paths are measured against: the tokenspeed PR #968
 * backend falls back to the whole operation done unfused whenever it declines (Summary (AI)), and
 * its performance figures compare against that. It moves 2 (n + 6) m hidden bytes instead of
 * 2 (n + 3) m hidden.
 * Arguments, conventions and errors as for fused_ar_rmsnorm (no path argument).
 */
int fused_ar_unfused_rmsnorm(const fa_bf16 *const *inputs, int n, const fa_bf16 *residual,
                             const fa_bf16 *weight, float eps, int m, int hidden,
                             fa_bf16 *residual_out, fa_bf16 *out, hipStream_t stream);

/*
 * fused_ar_rmsnorm_split - the one-stage result with every row cut into slices on separate
 * workgroups, so that a few rows still spread over many CUs, in two kernels: the first reduces,
 * adds the residual, writes residual_out and stores each slice's square-sum in `workspace`; the
 * second sums a row's slice square-sums in slice order and normalises each slice. residual_out is
 * bit-identical to fused_ar_rmsnorm's; out is deterministic and within the same 1-ulp band (its
 * square-sum is grouped by slice). The pages do not describe this form: it applies the reasoning
 * of aiter PR #3817 (Technical Details > 2stage > stage-1 launch config: more workgroups give small
 * problems more CUs) to the one-stage row. Measured on MI355X (N = 8, calls in a HIP graph): faster
 * than fused_ar_rmsnorm from hidden 16384 at m <= 32 (7.6 -> 4.4-4.5 us at hidden 32768, m = 1), slower
 * at hidden <= 7168 and at m = 128, since its second launch costs about a kernel launch.
 *
 *   splits     slices per row, 1..64 (capped at hidden / 8, so that no slice is empty); 0 = one
 *              slice per 256 packs of 8 elements. FUSED_AR_ERR_SHAPE if a slice would need more
 *              than 1024 threads (one pack per thread); FUSED_AR_ERR_INVALID outside 0..64.
 *   workspace  device buffer of at least fused_ar_split_workspace_bytes(m, hidden, splits) bytes,
 *              16-byte aligned, overlapping no other buffer; its contents are overwritten and need
 *              no initial value. Calls that share a workspace must be ordered (one stream).
 *   Other arguments, conventions and errors as for fused_ar_rmsnorm with the one-stage path; the
 *   workspace is checked after the other buffers (null or too small: FUSED_AR_ERR_INVALID,
 *   misaligned: FUSED_AR_ERR_ALIGN, overlapping: FUSED_AR_ERR_ALIAS).
 */
int fused_ar_rmsnorm_split(const fa_bf16 *const *inputs, int n, const fa_bf16 *residual,
                           const fa_bf16 *weight, float eps, int m, int hidden,
                           fa_bf16 *residual_out, fa_bf16 *out, int splits, void *workspace,
                           size_t workspace_bytes, hipStream_t stream);

/* fused_ar_split_workspace_bytes - the workspace fused_ar_rmsnorm_split needs for these scalars
 * (m * slices * 4 bytes); 0 when m == 0 or the scalars are invalid. */
size_t fused_ar_split_workspace_bytes(int m, int hidden, int splits);

/* Floats in the library's static scratch (256 KiB per GPU): fused_ar_rmsnorm_split_static takes
 * calls with m * slices up to this many. */
#define FUSED_AR_STATIC_SCRATCH_FLOATS 65536

/*
 * fused_ar_rmsnorm_split_static - fused_ar_rmsnorm_split without a workspace argument, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc. The slice square-sums go to a fixed device array of the library,
 * FUSED_AR_STATIC_SCRATCH_FLOATS floats, of which each GPU the library runs on holds its own copy
 * until the process ends; the call itself allocates nothing (no hipMalloc, no hipFree). The first
 * call on a device looks up that device's copy (hipGetSymbolAddress, with the device current);
 * callers that will capture it make one call on that device before capturing (tested: captured
 * calls replayed with eager calls of other shapes in between give the eager result).
 *   Limit: m * slices <= FUSED_AR_STATIC_SCRATCH_FLOATS (slices as fused_ar_split_workspace_bytes
 *   counts them: m <= 16384 at hidden 7168, m <= 4096 at hidden 32768, with the default slices);
 *   larger calls return FUSED_AR_ERR_SCRATCH and launch nothing.
 *   Sharing: every call on one GPU uses the same array, and it keeps the last call's contents
 *   (each call writes every slot it reads before reading it, so nothing needs clearing). Calls on
 *   one GPU that may run at the same time - on streams not ordered with one another - race on it
 *   and must not be made; calls ordered on one stream are safe.
 * Results are bit-identical to fused_ar_rmsnorm_split with the same arguments and splits. Other
 * arguments, conventions and errors as for fused_ar_rmsnorm_split (no workspace checks).
 */
int fused_ar_rmsnorm_split_static(const fa_bf16 *const *inputs, int n, const fa_bf16 *residual,
                                  const fa_bf16 *weight, float eps, int m, int hidden,
                                  fa_bf16 *residual_out, fa_bf16 *out, int splits,
                                  hipStream_t stream);

/* Options of fused_ar_rmsnorm_ex: alternative kernel designs, for comparison and tuning. */
enum {
    FUSED_AR_WAVE_DPP = 0,       /* wave reduction by a DPP butterfly (the default) */
    FUSED_AR_WAVE_BPERMUTE = 1,  /* wave reduction by a ds_bpermute XOR butterfly: the design the
                                    DPP tree replaced (aiter PR #3817, Technical Details > 1stage) */
    FUSED_AR_STAGE1_FLAT = 0,    /* stage 1: one thread per pack, no LDS, no barrier (the default) */
    FUSED_AR_STAGE1_LDS = 1      /* stage 1: one wave per input staging a tile through LDS, one
                                    barrier: the one-wave-per-rank design the flat reduce replaced
                                    (aiter PR #3817, Technical Details > 2stage > reduce-scatter) */
};

enum {
    FUSED_AR_LOAD_AUTO = 0,    /* ordinary loads when a call reads at most 128 MiB (its inputs may
                                  still be in the L2s or the 256 MB Infinity Cache), non-temporal
                                  loads above (inputs streamed from HBM) */
    FUSED_AR_LOAD_CACHED = 1,  /* always ordinary loads */
    FUSED_AR_LOAD_STREAM = 2   /* always non-temporal loads */
};

/* Where the two-stage path adds the residual (fused_ar_options.residual_stage).
 * - STAGE2, the split of aiter PR #3817 (Technical Details > 2stage): stage 1 stores the reduced
 *   rows (bf16) into `out` as its scratch, stage 2 reads them back, adds the residual, writes
 *   residual_out and normalises: 2 (n + 5) m hidden bytes moved.
 * - STAGE1: stage 1 reduces, adds the residual and writes residual_out; stage 2 is a plain
 *   RMSNorm of residual_out: 2 (n + 4) m hidden bytes, no scratch. Bit-identical to STAGE2 (the
 *   same roundings in the same order). On one GPU this is the faster split (by 5-10 % at the
 *   bandwidth sizes). Across GPUs the pages keep the reduced rows in a buffer registered for
 *   peer stores, which the caller's residual_out need not be.
 * - AUTO: STAGE1, except with the LDS-staged stage 1 or with chunks of rows, which exist only for
 *   STAGE2. STAGE1 together with either of those: FUSED_AR_ERR_INVALID. */
enum {
    FUSED_AR_RESIDUAL_AUTO = 0,
    FUSED_AR_RESIDUAL_STAGE2 = 1,
    FUSED_AR_RESIDUAL_STAGE1 = 2
};

/* How the two-stage path runs when it is cut into chunks of rows (fused_ar_options.stage_rows):
 * each chunk's stage 1 stores its reduced rows into `out` and its stage 2 reads them back soon
 * after, while they may still be in the L2s or the Infinity Cache, instead of after the whole
 * call's stage 1. */
enum {
    FUSED_AR_CHUNKS_AUTO = 0,        /* the library's choice */
    FUSED_AR_CHUNKS_SEQUENTIAL = 1,  /* stage 1 then stage 2 of each chunk in turn (two launches
                                        per chunk) */
    FUSED_AR_CHUNKS_PIPELINED = 2    /* one launch per chunk boundary: stage 2 of chunk c and
                                        stage 1 of chunk c + 1 on separate workgroups of one
                                        launch */
};

typedef struct {
    int wave_reduce;       /* FUSED_AR_WAVE_DPP or FUSED_AR_WAVE_BPERMUTE */
    int stage1;            /* FUSED_AR_STAGE1_FLAT or FUSED_AR_STAGE1_LDS */
    int stage1_block;      /* threads per workgroup of the flat kernels: 0 = by size, 256 (aiter
                              PR #3817, 2stage > stage-1 launch config) below 2^20 packs and 512
                              from there on; else a multiple of 64 in [64, 1024] */
    int packs_per_thread;  /* row kernels: 0 = automatic, else 1, 2 or 4 (FUSED_AR_ERR_SHAPE if the
                              row then needs more than 1024 threads) */
    int load_policy;       /* FUSED_AR_LOAD_AUTO, FUSED_AR_LOAD_CACHED or FUSED_AR_LOAD_STREAM: how
                              the inputs and the residual are loaded; streaming calls of more than
                              1024 rows also cap the row workgroups per CU and pick their packs
                              per thread (see fused_ar_rmsnorm_ex for what that does to `out`) */
    int stage_rows;        /* two-stage path: rows per chunk, 1..2^20; 0 = automatic; -1 = the
                              whole call as one chunk */
    int schedule;          /* two-stage path in chunks: FUSED_AR_CHUNKS_AUTO, _SEQUENTIAL or
                              _PIPELINED */
    int residual_stage;    /* two-stage path: where the residual is added, FUSED_AR_RESIDUAL_AUTO,
                              _STAGE2 or _STAGE1 (see the enum above) */
} fused_ar_options;

/*
 * fused_ar_rmsnorm_ex - fused_ar_rmsnorm with `options` (NULL = the defaults, identical to
 * fused_ar_rmsnorm); `path` may also be FUSED_AR_PATH_UNFUSED. Every option combination gives
 * bit-identical residual_out; `out` is bit-identical too unless the row geometry changes - by
 * packs_per_thread, or by load_policy on calls of more than 1024 rows, whose streaming form takes
 * its own packs per thread - and with it the order of the row's square-sum (then within the same
 * 1-ulp band). Bad options: FUSED_AR_ERR_INVALID. Otherwise as fused_ar_rmsnorm.
 */
int fused_ar_rmsnorm_ex(const fa_bf16 *const *inputs, int n, const fa_bf16 *residual,
                        const fa_bf16 *weight, float eps, int m, int hidden, fa_bf16 *residual_out,
                        fa_bf16 *out, int path, const fused_ar_options *options,
                        hipStream_t stream);

/*
 * fused_ar_rmsnorm_check - the argument checks of fused_ar_rmsnorm alone, with the same arguments
 * (no stream): returns the status fused_ar_rmsnorm would return before launching anything
 * (FUSED_AR_OK if it would launch). Makes no HIP call. A preflight for callers that must decide
 * on a fallback before work is enqueued (the concern behind the decline/fallback review threads
 * of tokenspeed PR #968).
 */
int fused_ar_rmsnorm_check(const fa_bf16 *const *inputs, int n, const fa_bf16 *residual,
                           const fa_bf16 *weight, float eps, int m, int hidden,
                           const fa_bf16 *residual_out, const fa_bf16 *out, int path);

/*
 * fused_ar_reduce - the reduce alone, the two-stage path's first kernel, flat as in aiter PR #3817,
 * Technical Details > 2stage > reduce-scatter: one thread per 8-element pack,
 * fp32 sum over the n inputs in array order, one bf16 store; no LDS, no workgroup barrier.
 *
 *   inputs   host array of n device pointers, each m * hidden bf16 (contiguous).
 *   n        1..FUSED_AR_MAX_INPUTS.
 *   m, hidden  m >= 0 (0 launches nothing); hidden > 0 and a multiple of 8 (no upper bound).
 *   reduced  device m * hidden bf16, written; must not overlap any input.
 *   stream   HIP stream.
 * Errors as for fused_ar_rmsnorm. All pointers 16-byte aligned.
 */
int fused_ar_reduce(const fa_bf16 *const *inputs, int n, int m, int hidden, fa_bf16 *reduced,
                    hipStream_t stream);

/*
 * fused_ar_auto_path - the path FUSED_AR_PATH_AUTO takes, tuned on one MI355X where all n partial
 * sums are in local HBM. With R = 2 (n + 1) hidden, the bytes a row reads (n inputs and the
 * residual): the two-stage path for m <= 48 when R >= 512 KiB, for m <= 40 when R >= 432 KiB and
 * for m <= 16 when R >= 336 KiB; the one-stage path otherwise. Measured over n = 2..8,
 * hidden = 2880..32768, m = 1..8192: the one-stage path is faster everywhere except for a few rows
 * too long for one CU each (from n = 8, hidden >= 20480 or n = 4, hidden = 32768 at small m),
 * where the two-stage path's flat first kernel spreads the reads over every CU.
 * Returns 1 or 2, or FUSED_AR_ERR_INVALID for n outside [1, 8], m < 0 or hidden <= 0.
 */
int fused_ar_auto_path(int n, int m, int hidden);

/*
 * fused_ar_auto_path_tp - the selection rule of the pages for a tensor-parallel group whose
 * partial sums sit on n GPUs: one-stage for m <= 32 when n <= 4 and for m <= 16 when n > 4,
 * two-stage above (aiter PR #3817, Test Results: the thresholds for TP4 and TP8, extended to other
 * n by n <= 4 / n > 4). Those thresholds weigh the link traffic of reading every peer in full
 * (one-stage) against a reduce-scatter and gather (two-stage), which one GPU does not have; the
 * rule is kept for the multi-GPU form of this path. Returns 1 or 2, or FUSED_AR_ERR_INVALID for n
 * outside [1, 8] or m < 0 (`hidden` is not used).
 */
int fused_ar_auto_path_tp(int n, int m, int hidden);

/* One kernel launch of a call, as fused_ar_describe_launch reports it. */
typedef struct {
    char name[32];        /* kernel name: "onestage", "stage1_reduce", "stage1_reduce_lds",
                             "stage_pipe" (stage 2 of one chunk with stage 1 of the next),
                             "stage1_reduce_residual", "stage2_norm", "stage2_rmsnorm",
                             "residual_add" or "rmsnorm" */
    unsigned grid;        /* workgroups per launch (the row kernels: one per row) */
    unsigned block;       /* threads per workgroup (a multiple of 64) */
    unsigned per_thread;  /* 8-element packs each thread handles per row (1 in flat kernels) */
    unsigned launches;    /* launches of this kernel per call: rows come in launches of at most
                             2^20 workgroups, flat kernels' packs in launches of at most 2^30 */
    unsigned streaming;   /* 1: non-temporal loads of the inputs; 0: ordinary loads */
    unsigned lds_bytes;   /* LDS reserved per workgroup beyond the kernel's own, to cap the
                             workgroups resident per CU (row kernels of long streaming calls) */
} fused_ar_kernel_launch;

typedef struct {
    int path;                       /* resolved path: 1, 2 or 3 (unfused) */
    int kernels;                    /* kernels per call: 1, 2 or 3; 0 when m == 0 */
    fused_ar_kernel_launch launch[3];
} fused_ar_launch_plan;

/*
 * fused_ar_describe_launch - the kernels, grids and workgroup sizes fused_ar_rmsnorm (or, for
 * FUSED_AR_PATH_UNFUSED, fused_ar_unfused_rmsnorm) would use for (n, m, hidden, path), without
 * launching anything. For benchmarks and tests. Returns FUSED_AR_OK, or the error the call would
 * give for these scalars. fused_ar_describe_launch_ex does the same for fused_ar_rmsnorm_ex.
 */
int fused_ar_describe_launch(int n, int m, int hidden, int path, fused_ar_launch_plan *plan);
int fused_ar_describe_launch_ex(int n, int m, int hidden, int path,
                                const fused_ar_options *options, fused_ar_launch_plan *plan);

/* fused_ar_strerror - a static, human-readable description of a status code. Never NULL. */
const char *fused_ar_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* FUSED_AR_H */
