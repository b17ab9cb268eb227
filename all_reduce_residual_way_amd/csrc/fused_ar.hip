// fused_ar.hip - host side of libfused_ar.so: argument checks, path choice, launch geometry and
// the extern "C" entry points declared in include/fused_ar.h.
#include "fused_ar.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#include "kernels.h"

namespace {

using fa::FlatArgs;
using fa::RowArgs;

constexpr int kPackElems = 8;
constexpr int kMaxBlock = 1024;
constexpr unsigned kFlatBlock = 256;              // stage-1 workgroup (aiter PR #3817, 2stage >
                                                  // stage-1 launch config)
constexpr size_t kFlatMaxGrid = size_t(1) << 22;  // beyond this the flat kernel strides
constexpr int kRowsPerLaunch = 1 << 20;           // taller problems take several launches

struct Span {
    uintptr_t lo, hi;  // [lo, hi)
};

bool make_span(const void *p, size_t bytes, Span *s)
{
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    if (lo > UINTPTR_MAX - bytes)
        return false;
    *s = {lo, lo + bytes};
    return true;
}

bool overlaps(const Span &a, const Span &b) { return a.lo < b.hi && b.lo < a.hi; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Packs per thread and threads per workgroup of the row kernel for m rows of `packs` packs.
// Few rows (m <= kWideRowsMaxM): one pack per thread where the row fits in 1024 threads, so each
// thread issues all its loads at once and a row costs one memory round trip (latency). Many rows:
// at least two packs per thread where rows are wider than 512 packs, i.e. smaller workgroups,
// more of them resident per CU, and the workgroup barriers of different rows overlap
// (bandwidth). Packs per thread grow (1, 2, 4) until the row fits in 1024 threads; the thread
// count is rounded up to whole waves. FUSED_AR_MAX_HIDDEN = 4 * 1024 * 8 elements.
constexpr int kWideRowsMaxM = 256;

void row_geometry(int packs, int m, int *ppt, int *threads)
{
    int k = (m > kWideRowsMaxM && packs > 512) ? 2 : 1;
    while (k < 4 && (packs + k - 1) / k > kMaxBlock)
        k *= 2;
    *ppt = k;
    const int t = (packs + k - 1) / k;
    *threads = (t + 63) / 64 * 64;
}

template <int N>
const void *row_kernel_n(int ppt)
{
    switch (ppt) {
    case 1: return reinterpret_cast<const void *>(&fa::k_rows<N, 1>);
    case 2: return reinterpret_cast<const void *>(&fa::k_rows<N, 2>);
    case 4: return reinterpret_cast<const void *>(&fa::k_rows<N, 4>);
    default: return nullptr;
    }
}

const void *row_kernel(int n, int ppt)
{
    switch (n) {
    case 1: return row_kernel_n<1>(ppt);
    case 2: return row_kernel_n<2>(ppt);
    case 3: return row_kernel_n<3>(ppt);
    case 4: return row_kernel_n<4>(ppt);
    case 5: return row_kernel_n<5>(ppt);
    case 6: return row_kernel_n<6>(ppt);
    case 7: return row_kernel_n<7>(ppt);
    case 8: return row_kernel_n<8>(ppt);
    default: return nullptr;
    }
}

const void *flat_kernel(int n)
{
    switch (n) {
    case 1: return reinterpret_cast<const void *>(&fa::k_flat_reduce<1>);
    case 2: return reinterpret_cast<const void *>(&fa::k_flat_reduce<2>);
    case 3: return reinterpret_cast<const void *>(&fa::k_flat_reduce<3>);
    case 4: return reinterpret_cast<const void *>(&fa::k_flat_reduce<4>);
    case 5: return reinterpret_cast<const void *>(&fa::k_flat_reduce<5>);
    case 6: return reinterpret_cast<const void *>(&fa::k_flat_reduce<6>);
    case 7: return reinterpret_cast<const void *>(&fa::k_flat_reduce<7>);
    case 8: return reinterpret_cast<const void *>(&fa::k_flat_reduce<8>);
    default: return nullptr;
    }
}

unsigned flat_grid(size_t total_packs)
{
    size_t g = (total_packs + kFlatBlock - 1) / kFlatBlock;
    if (g > kFlatMaxGrid)
        g = kFlatMaxGrid;
    return static_cast<unsigned>(g);
}

unsigned rows_grid(int m) { return static_cast<unsigned>(m < kRowsPerLaunch ? m : kRowsPerLaunch); }

unsigned rows_launches(int m) { return static_cast<unsigned>((m + kRowsPerLaunch - 1) / kRowsPerLaunch); }

int check_scalars(int n, int m, int hidden, float eps, int path, bool bounded_hidden)
{
    if (n < 1 || n > FUSED_AR_MAX_INPUTS || m < 0 || hidden <= 0)
        return FUSED_AR_ERR_INVALID;
    if (!(eps >= 0.0f) || !isfinite(eps))
        return FUSED_AR_ERR_INVALID;
    if (path < FUSED_AR_PATH_AUTO || path > FUSED_AR_PATH_TWOSTAGE)
        return FUSED_AR_ERR_INVALID;
    if (hidden % kPackElems != 0)
        return FUSED_AR_ERR_SHAPE;
    if (bounded_hidden && hidden > FUSED_AR_MAX_HIDDEN)
        return FUSED_AR_ERR_SHAPE;
    return FUSED_AR_OK;
}

int launch(const void *kernel, unsigned grid, unsigned block, void *args, hipStream_t stream)
{
    void *params[] = {args};
    const hipError_t e = hipLaunchKernel(kernel, dim3(grid), dim3(block), params, 0, stream);
    return e == hipSuccess ? FUSED_AR_OK : static_cast<int>(e);
}

// One workgroup per row, at most kRowsPerLaunch rows per launch; later launches start
// kRowsPerLaunch rows further into every [m, hidden] buffer.
int run_rows(const RowArgs &args, int n, int m, int packs, hipStream_t stream)
{
    int ppt, threads;
    row_geometry(packs, m, &ppt, &threads);
    const void *kernel = row_kernel(n, ppt);
    for (int first = 0; first < m; first += kRowsPerLaunch) {
        const int rows = m - first < kRowsPerLaunch ? m - first : kRowsPerLaunch;
        const size_t skip = (size_t)first * (size_t)packs;  // in packs
        RowArgs a = args;
        for (int i = 0; i < n; ++i)
            a.in[i] += skip;
        a.residual += skip;
        a.residual_out += skip;
        a.out += skip;
        const int rc = launch(kernel, static_cast<unsigned>(rows), threads, &a, stream);
        if (rc != FUSED_AR_OK)
            return rc;
    }
    return FUSED_AR_OK;
}

int run_flat(const fa_bf16 *const *inputs, int n, size_t total_packs, fa_bf16 *reduced,
             hipStream_t stream)
{
    FlatArgs a{};
    for (int i = 0; i < n; ++i)
        a.in[i] = reinterpret_cast<const fa::u32x4 *>(inputs[i]);
    a.out = reinterpret_cast<fa::u32x4 *>(reduced);
    a.total_packs = total_packs;
    return launch(flat_kernel(n), flat_grid(total_packs), kFlatBlock, &a, stream);
}

}  // namespace

extern "C" int fused_ar_auto_path(int n, int m, int hidden)
{
    (void)hidden;
    if (n < 1 || n > FUSED_AR_MAX_INPUTS || m < 0)
        return FUSED_AR_ERR_INVALID;
    const int one_stage_max_m = n <= 4 ? 32 : 16;
    return m <= one_stage_max_m ? FUSED_AR_PATH_ONESTAGE : FUSED_AR_PATH_TWOSTAGE;
}

extern "C" int fused_ar_rmsnorm_check(const fa_bf16 *const *inputs, int n,
                                      const fa_bf16 *residual, const fa_bf16 *weight, float eps,
                                      int m, int hidden, const fa_bf16 *residual_out,
                                      const fa_bf16 *out, int path)
{
    int rc = check_scalars(n, m, hidden, eps, path, true);
    if (rc != FUSED_AR_OK || m == 0)
        return rc;
    if (inputs == nullptr || residual == nullptr || weight == nullptr || residual_out == nullptr ||
        out == nullptr)
        return FUSED_AR_ERR_INVALID;
    for (int i = 0; i < n; ++i)
        if (inputs[i] == nullptr)
            return FUSED_AR_ERR_INVALID;

    const size_t plane = (size_t)m * (size_t)hidden * sizeof(fa_bf16);
    Span in_s[FUSED_AR_MAX_INPUTS], res_s, w_s, ro_s, out_s;
    for (int i = 0; i < n; ++i)
        if (!make_span(inputs[i], plane, &in_s[i]))
            return FUSED_AR_ERR_INVALID;
    if (!make_span(residual, plane, &res_s) ||
        !make_span(weight, (size_t)hidden * sizeof(fa_bf16), &w_s) ||
        !make_span(residual_out, plane, &ro_s) || !make_span(out, plane, &out_s))
        return FUSED_AR_ERR_INVALID;

    for (int i = 0; i < n; ++i)
        if (!aligned16(inputs[i]))
            return FUSED_AR_ERR_ALIGN;
    if (!aligned16(residual) || !aligned16(weight) || !aligned16(residual_out) || !aligned16(out))
        return FUSED_AR_ERR_ALIGN;

    for (int i = 0; i < n; ++i)
        if (overlaps(out_s, in_s[i]) || overlaps(ro_s, in_s[i]))
            return FUSED_AR_ERR_ALIAS;
    if (overlaps(out_s, res_s) || overlaps(out_s, w_s) || overlaps(out_s, ro_s) ||
        overlaps(ro_s, w_s))
        return FUSED_AR_ERR_ALIAS;
    if (overlaps(ro_s, res_s) && ro_s.lo != res_s.lo)
        return FUSED_AR_ERR_ALIAS;
    return FUSED_AR_OK;
}

extern "C" int fused_ar_rmsnorm(const fa_bf16 *const *inputs, int n, const fa_bf16 *residual,
                                const fa_bf16 *weight, float eps, int m, int hidden,
                                fa_bf16 *residual_out, fa_bf16 *out, int path, hipStream_t stream)
{
    int rc = fused_ar_rmsnorm_check(inputs, n, residual, weight, eps, m, hidden, residual_out, out,
                                    path);
    if (rc != FUSED_AR_OK || m == 0)
        return rc;

    if (path == FUSED_AR_PATH_AUTO)
        path = fused_ar_auto_path(n, m, hidden);

    const int packs = hidden / kPackElems;
    RowArgs a{};
    a.residual = reinterpret_cast<const fa::u32x4 *>(residual);
    a.weight = reinterpret_cast<const fa::u32x4 *>(weight);
    a.residual_out = reinterpret_cast<fa::u32x4 *>(residual_out);
    a.out = reinterpret_cast<fa::u32x4 *>(out);
    a.eps = eps;
    a.hidden = static_cast<float>(hidden);
    a.packs = packs;

    if (path == FUSED_AR_PATH_ONESTAGE) {
        for (int i = 0; i < n; ++i)
            a.in[i] = reinterpret_cast<const fa::u32x4 *>(inputs[i]);
        return run_rows(a, n, m, packs, stream);
    }

    // Two-stage: the flat reduce writes the reduced rows into `out`, then the row kernel with a
    // single input reads them back from there and overwrites them with the normalised rows.
    rc = run_flat(inputs, n, (size_t)m * (size_t)packs, out, stream);
    if (rc != FUSED_AR_OK)
        return rc;
    a.in[0] = reinterpret_cast<const fa::u32x4 *>(out);
    return run_rows(a, 1, m, packs, stream);
}

extern "C" int fused_ar_reduce(const fa_bf16 *const *inputs, int n, int m, int hidden,
                               fa_bf16 *reduced, hipStream_t stream)
{
    int rc = check_scalars(n, m, hidden, 0.0f, FUSED_AR_PATH_AUTO, false);
    if (rc != FUSED_AR_OK)
        return rc;
    if (m == 0)
        return FUSED_AR_OK;
    if (inputs == nullptr || reduced == nullptr)
        return FUSED_AR_ERR_INVALID;
    for (int i = 0; i < n; ++i)
        if (inputs[i] == nullptr)
            return FUSED_AR_ERR_INVALID;
    const size_t total_packs = (size_t)m * (size_t)(hidden / kPackElems);
    const size_t plane = total_packs * 16;
    Span red_s, in_s[FUSED_AR_MAX_INPUTS];
    if (!make_span(reduced, plane, &red_s))
        return FUSED_AR_ERR_INVALID;
    for (int i = 0; i < n; ++i)
        if (!make_span(inputs[i], plane, &in_s[i]))
            return FUSED_AR_ERR_INVALID;
    for (int i = 0; i < n; ++i)
        if (!aligned16(inputs[i]))
            return FUSED_AR_ERR_ALIGN;
    if (!aligned16(reduced))
        return FUSED_AR_ERR_ALIGN;
    for (int i = 0; i < n; ++i)
        if (overlaps(red_s, in_s[i]))
            return FUSED_AR_ERR_ALIAS;
    return run_flat(inputs, n, total_packs, reduced, stream);
}

extern "C" int fused_ar_describe_launch(int n, int m, int hidden, int path,
                                        fused_ar_launch_plan *plan)
{
    const int rc = check_scalars(n, m, hidden, 0.0f, path, true);
    if (rc != FUSED_AR_OK)
        return rc;
    if (plan == nullptr)
        return FUSED_AR_ERR_INVALID;
    memset(plan, 0, sizeof(*plan));
    if (path == FUSED_AR_PATH_AUTO)
        path = fused_ar_auto_path(n, m, hidden);
    plan->path = path;
    if (m == 0)
        return FUSED_AR_OK;
    const int packs = hidden / kPackElems;
    int ppt, threads;
    row_geometry(packs, m, &ppt, &threads);
    fused_ar_kernel_launch rows{};
    rows.grid = rows_grid(m);
    rows.block = static_cast<unsigned>(threads);
    rows.per_thread = static_cast<unsigned>(ppt);
    rows.launches = rows_launches(m);
    if (path == FUSED_AR_PATH_ONESTAGE) {
        plan->kernels = 1;
        strcpy(rows.name, "onestage");
        plan->launch[0] = rows;
    } else {
        plan->kernels = 2;
        fused_ar_kernel_launch flat{};
        strcpy(flat.name, "stage1_reduce");
        const size_t total = (size_t)m * (size_t)packs;
        flat.grid = flat_grid(total);
        flat.block = kFlatBlock;
        const size_t covered = (size_t)flat.grid * kFlatBlock;
        flat.per_thread = static_cast<unsigned>((total + covered - 1) / covered);
        flat.launches = 1;
        strcpy(rows.name, "stage2_norm");
        plan->launch[0] = flat;
        plan->launch[1] = rows;
    }
    return FUSED_AR_OK;
}

extern "C" const char *fused_ar_strerror(int status)
{
    switch (status) {
    case FUSED_AR_OK: return "success";
    case FUSED_AR_ERR_INVALID: return "invalid argument (null pointer, n, m, hidden, eps or path out of range)";
    case FUSED_AR_ERR_SHAPE: return "unsupported shape (hidden must be a multiple of 8 and at most 32768)";
    case FUSED_AR_ERR_ALIGN: return "a device pointer is not 16-byte aligned";
    case FUSED_AR_ERR_ALIAS: return "forbidden overlap between output and other buffers";
    default: break;
    }
    if (status > 0)
        return hipGetErrorString(static_cast<hipError_t>(status));
    return "unknown status";
}
