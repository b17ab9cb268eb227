// fused_ar.hip - host side of libfused_ar.so: argument checks, path choice, launch plans and the
// extern "C" entry points declared in include/fused_ar.h.
#include "fused_ar.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "kernels.h"

namespace {

using fa::FlatArgs;
using fa::RowArgs;
using fa::u32x4;

constexpr int kPackElems = 8;
constexpr int kMaxBlock = 1024;
// Workgroup of the flat kernels: 256 threads (aiter PR #3817, 2stage > stage-1 launch config:
// more workgroups give small problems more CUs), 512 from kFlatLargePacks packs on, where there is
// parallelism to spare and half as many workgroups to dispatch make path 2 up to 3 % faster
// (measured on MI355X: N = 8, m = 4096 and 8192; within 1 % at N = 4 and m <= 1024).
constexpr unsigned kFlatBlock = 256;
constexpr unsigned kFlatBlockLarge = 512;
constexpr size_t kFlatLargePacks = size_t(1) << 20;
constexpr size_t kFlatPacksPerLaunch = size_t(1) << 30;  // more packs take several launches
constexpr int kRowsPerLaunch = 1 << 20;           // taller problems take several launches
constexpr int kPathUnfusedPlan = 3;               // internal plan id of the unfused sequence

// ------------------------------------------------------------------------------------ checks

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

// The pointer checks of fused_ar_rmsnorm (m > 0): nulls, alignment, forbidden overlaps.
int check_buffers(const fa_bf16 *const *inputs, int n, const fa_bf16 *residual,
                  const fa_bf16 *weight, int m, int hidden, const fa_bf16 *residual_out,
                  const fa_bf16 *out)
{
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

// ------------------------------------------------------------------------------------ plans

struct Options {
    bool bpermute;        // wave reduction by ds_bpermute instead of DPP
    bool lds_stage1;      // LDS-staged wave-per-input stage 1 instead of the flat reduce
    unsigned flat_block;  // workgroup of the flat kernels; 0 = by size (flat_block_for)
    int ppt;              // packs per thread of the row kernels; 0 = automatic
    int load_policy;      // FUSED_AR_LOAD_AUTO, _CACHED or _STREAM
    int stage_rows;       // two-stage path: rows per chunk; 0 = automatic, -1 = one chunk
    int schedule;         // FUSED_AR_CHUNKS_AUTO, _SEQUENTIAL or _PIPELINED
    int residual_stage;   // two-stage path: FUSED_AR_RESIDUAL_AUTO, _STAGE2 or _STAGE1
};

constexpr Options kDefaultOptions = {false, false, 0, 0, FUSED_AR_LOAD_AUTO, 0,
                                     FUSED_AR_CHUNKS_AUTO, FUSED_AR_RESIDUAL_AUTO};

unsigned flat_block_for(const Options &o, size_t total_packs)
{
    if (o.flat_block != 0)
        return o.flat_block;
    return total_packs >= kFlatLargePacks ? kFlatBlockLarge : kFlatBlock;
}

// Automatic load policy. Non-temporal loads are 6-12 % faster when the inputs come from HBM, and
// ordinary loads 3-35 % faster when they are still in the L2s (8 x 4 MB) or the 256 MB Infinity
// Cache (measured on MI355X, N = 4 and 8, m = 1..512). Inputs written by the kernel that ran just
// before can only still be cached when a call reads well under the Infinity Cache's capacity, so
// calls that read at most half of it use ordinary loads and larger ones stream.
constexpr uint64_t kStreamMinReadBytes = uint64_t(128) << 20;

bool use_stream(const Options &o, int n, int m, int hidden)
{
    if (o.load_policy != FUSED_AR_LOAD_AUTO)
        return o.load_policy == FUSED_AR_LOAD_STREAM;
    const uint64_t read = 2ull * (uint64_t)(n + 1) * (uint64_t)m * (uint64_t)hidden;
    return read > kStreamMinReadBytes;
}

int read_options(const fused_ar_options *o, Options *out)
{
    *out = kDefaultOptions;
    if (o == nullptr)
        return FUSED_AR_OK;
    if ((o->wave_reduce != FUSED_AR_WAVE_DPP && o->wave_reduce != FUSED_AR_WAVE_BPERMUTE) ||
        (o->stage1 != FUSED_AR_STAGE1_FLAT && o->stage1 != FUSED_AR_STAGE1_LDS))
        return FUSED_AR_ERR_INVALID;
    if (o->stage1_block != 0 &&
        (o->stage1_block < 64 || o->stage1_block > kMaxBlock || o->stage1_block % 64 != 0))
        return FUSED_AR_ERR_INVALID;
    if (o->packs_per_thread != 0 && o->packs_per_thread != 1 && o->packs_per_thread != 2 &&
        o->packs_per_thread != 4)
        return FUSED_AR_ERR_INVALID;
    if (o->load_policy != FUSED_AR_LOAD_AUTO && o->load_policy != FUSED_AR_LOAD_CACHED &&
        o->load_policy != FUSED_AR_LOAD_STREAM)
        return FUSED_AR_ERR_INVALID;
    if (o->stage_rows < -1 || o->stage_rows > kRowsPerLaunch)
        return FUSED_AR_ERR_INVALID;
    if (o->schedule != FUSED_AR_CHUNKS_AUTO && o->schedule != FUSED_AR_CHUNKS_SEQUENTIAL &&
        o->schedule != FUSED_AR_CHUNKS_PIPELINED)
        return FUSED_AR_ERR_INVALID;
    if (o->residual_stage != FUSED_AR_RESIDUAL_AUTO &&
        o->residual_stage != FUSED_AR_RESIDUAL_STAGE2 && o->residual_stage != FUSED_AR_RESIDUAL_STAGE1)
        return FUSED_AR_ERR_INVALID;
    // the residual add in stage 1 has only the flat, unchunked form
    if (o->residual_stage == FUSED_AR_RESIDUAL_STAGE1 &&
        (o->stage1 == FUSED_AR_STAGE1_LDS || o->stage_rows > 0))
        return FUSED_AR_ERR_INVALID;
    out->bpermute = o->wave_reduce == FUSED_AR_WAVE_BPERMUTE;
    out->lds_stage1 = o->stage1 == FUSED_AR_STAGE1_LDS;
    out->flat_block = static_cast<unsigned>(o->stage1_block);
    out->ppt = o->packs_per_thread;
    out->load_policy = o->load_policy;
    out->stage_rows = o->stage_rows;
    out->schedule = o->schedule;
    out->residual_stage = o->residual_stage;
    return FUSED_AR_OK;
}

// Packs per thread and threads per workgroup of the row kernel for m rows of `packs` packs.
// Calls that read from the caches, or that have few rows: one pack per thread where the row fits
// in 1024 threads, so that each thread issues all its loads at once and a row costs one memory
// round trip; except that for 256 < m <= 1024 rows wider than 512 packs two packs per thread
// (half-size workgroups, twice as many resident per CU) are up to 7 % faster (measured on MI355X,
// N = 4 and 8, hidden 4096-8192).
// Long calls that stream from HBM (`capped`: at most two row workgroups per CU, see kRowCapLds)
// go best with fewer threads per row, its packs taken in turn: two packs per thread for rows of
// 512-1024 packs and four above, one below (N = 8, cold, % of peak with one / two / four packs
// per thread: hidden 2880 79.7 / 77.4 / 73.7, 4096 77.2 / 80.0 / 76.3, 6144 73.7 / 75.7 / 77.2,
// 7168 75.8 / 76.4 / 75.6, 8192 75.8 / 77.4 / 76.0, 16384 - / 73.3 / 73.9).
// Packs per thread grow (1, 2, 4) until the row fits in 1024 threads; the thread count is
// rounded up to whole waves. FUSED_AR_MAX_HIDDEN = 4 * 1024 * 8 elements.
constexpr int kTwoPackMinM = 257;
constexpr int kTwoPackMaxM = 1024;

// Row workgroups resident per CU on long streaming calls. Small rows let up to five row
// workgroups reside per CU, about 1000 rows in flight, and HBM then serves the interleaved reads
// less well: capping the row kernel at two resident workgroups per CU (about 512 rows in flight)
// measured +4.0 points of peak at hidden 2880, +3.5 at 4096 and +1.3 at 5120 (N = 8, one pack per
// thread). The cap is a reservation of LDS the kernel does not use: 64 KiB of the CU's 160 KiB
// admits two workgroups, not three. It applies to calls that stream (cache-resident calls lose
// by it: -3.9 points at hidden 2880, m = 1000, warm) and have more than kTwoPackMaxM rows, so that
// the rows of the two-pack band stay resident in one round.
constexpr unsigned kRowCapLds = 64u * 1024u;

bool rows_capped(bool stream, int m) { return stream && m > kTwoPackMaxM; }

int row_geometry(int packs, int m, int forced_ppt, bool capped, int *ppt, int *threads)
{
    int k = forced_ppt;
    if (k == 0) {
        if (capped)
            k = packs > 1024 ? 4 : (packs >= 512 ? 2 : 1);
        else
            k = (m >= kTwoPackMinM && m <= kTwoPackMaxM && packs > 512) ? 2 : 1;
        while (k < 4 && (packs + k - 1) / k > kMaxBlock)
            k *= 2;
    } else if ((packs + k - 1) / k > kMaxBlock) {
        return FUSED_AR_ERR_SHAPE;  // the requested packs per thread do not fit the row
    }
    *ppt = k;
    const int t = (packs + k - 1) / k;
    *threads = (t + 63) / 64 * 64;
    return FUSED_AR_OK;
}

template <int N, bool kB, bool kR, bool kS>
const void *row_kernel_np(int ppt)
{
    switch (ppt) {
    case 1: return reinterpret_cast<const void *>(&fa::k_rows<N, 1, kB, kR, kS>);
    case 2: return reinterpret_cast<const void *>(&fa::k_rows<N, 2, kB, kR, kS>);
    case 4: return reinterpret_cast<const void *>(&fa::k_rows<N, 4, kB, kR, kS>);
    default: return nullptr;
    }
}

template <bool kB, bool kS>
const void *row_kernel_bs(int n, int ppt, bool residual)
{
    if (!residual)
        return n == 1 ? row_kernel_np<1, kB, false, kS>(ppt) : nullptr;
    switch (n) {
    case 1: return row_kernel_np<1, kB, true, kS>(ppt);
    case 2: return row_kernel_np<2, kB, true, kS>(ppt);
    case 3: return row_kernel_np<3, kB, true, kS>(ppt);
    case 4: return row_kernel_np<4, kB, true, kS>(ppt);
    case 5: return row_kernel_np<5, kB, true, kS>(ppt);
    case 6: return row_kernel_np<6, kB, true, kS>(ppt);
    case 7: return row_kernel_np<7, kB, true, kS>(ppt);
    case 8: return row_kernel_np<8, kB, true, kS>(ppt);
    default: return nullptr;
    }
}

const void *row_kernel(int n, int ppt, bool bpermute, bool residual, bool stream)
{
    if (bpermute)
        return stream ? row_kernel_bs<true, true>(n, ppt, residual)
                      : row_kernel_bs<true, false>(n, ppt, residual);
    return stream ? row_kernel_bs<false, true>(n, ppt, residual)
                  : row_kernel_bs<false, false>(n, ppt, residual);
}

template <bool kS>
const void *flat_kernel_s(int n)
{
    switch (n) {
    case 1: return reinterpret_cast<const void *>(&fa::k_flat_reduce<1, kS>);
    case 2: return reinterpret_cast<const void *>(&fa::k_flat_reduce<2, kS>);
    case 3: return reinterpret_cast<const void *>(&fa::k_flat_reduce<3, kS>);
    case 4: return reinterpret_cast<const void *>(&fa::k_flat_reduce<4, kS>);
    case 5: return reinterpret_cast<const void *>(&fa::k_flat_reduce<5, kS>);
    case 6: return reinterpret_cast<const void *>(&fa::k_flat_reduce<6, kS>);
    case 7: return reinterpret_cast<const void *>(&fa::k_flat_reduce<7, kS>);
    case 8: return reinterpret_cast<const void *>(&fa::k_flat_reduce<8, kS>);
    default: return nullptr;
    }
}

const void *flat_kernel(int n, bool stream)
{
    return stream ? flat_kernel_s<true>(n) : flat_kernel_s<false>(n);
}

template <bool kS>
const void *flat_residual_kernel_s(int n)
{
    switch (n) {
    case 1: return reinterpret_cast<const void *>(&fa::k_flat_residual<1, kS>);
    case 2: return reinterpret_cast<const void *>(&fa::k_flat_residual<2, kS>);
    case 3: return reinterpret_cast<const void *>(&fa::k_flat_residual<3, kS>);
    case 4: return reinterpret_cast<const void *>(&fa::k_flat_residual<4, kS>);
    case 5: return reinterpret_cast<const void *>(&fa::k_flat_residual<5, kS>);
    case 6: return reinterpret_cast<const void *>(&fa::k_flat_residual<6, kS>);
    case 7: return reinterpret_cast<const void *>(&fa::k_flat_residual<7, kS>);
    case 8: return reinterpret_cast<const void *>(&fa::k_flat_residual<8, kS>);
    default: return nullptr;
    }
}

const void *flat_residual_kernel(int n, bool stream)
{
    return stream ? flat_residual_kernel_s<true>(n) : flat_residual_kernel_s<false>(n);
}

template <int P, bool kS>
const void *pipe_kernel_ps(int n)
{
    switch (n) {
    case 1: return reinterpret_cast<const void *>(&fa::k_pipe<1, P, kS>);
    case 2: return reinterpret_cast<const void *>(&fa::k_pipe<2, P, kS>);
    case 3: return reinterpret_cast<const void *>(&fa::k_pipe<3, P, kS>);
    case 4: return reinterpret_cast<const void *>(&fa::k_pipe<4, P, kS>);
    case 5: return reinterpret_cast<const void *>(&fa::k_pipe<5, P, kS>);
    case 6: return reinterpret_cast<const void *>(&fa::k_pipe<6, P, kS>);
    case 7: return reinterpret_cast<const void *>(&fa::k_pipe<7, P, kS>);
    case 8: return reinterpret_cast<const void *>(&fa::k_pipe<8, P, kS>);
    default: return nullptr;
    }
}

template <bool kS>
const void *pipe_kernel_s(int n, int ppt)
{
    switch (ppt) {
    case 1: return pipe_kernel_ps<1, kS>(n);
    case 2: return pipe_kernel_ps<2, kS>(n);
    case 4: return pipe_kernel_ps<4, kS>(n);
    default: return nullptr;
    }
}

const void *pipe_kernel(int n, int ppt, bool stream)
{
    return stream ? pipe_kernel_s<true>(n, ppt) : pipe_kernel_s<false>(n, ppt);
}

template <bool kS>
const void *lds_kernel_s(int n)
{
    switch (n) {
    case 1: return reinterpret_cast<const void *>(&fa::k_stage1_lds<1, kS>);
    case 2: return reinterpret_cast<const void *>(&fa::k_stage1_lds<2, kS>);
    case 3: return reinterpret_cast<const void *>(&fa::k_stage1_lds<3, kS>);
    case 4: return reinterpret_cast<const void *>(&fa::k_stage1_lds<4, kS>);
    case 5: return reinterpret_cast<const void *>(&fa::k_stage1_lds<5, kS>);
    case 6: return reinterpret_cast<const void *>(&fa::k_stage1_lds<6, kS>);
    case 7: return reinterpret_cast<const void *>(&fa::k_stage1_lds<7, kS>);
    case 8: return reinterpret_cast<const void *>(&fa::k_stage1_lds<8, kS>);
    default: return nullptr;
    }
}

const void *lds_kernel(int n, bool stream)
{
    return stream ? lds_kernel_s<true>(n) : lds_kernel_s<false>(n);
}

template <bool kS>
const void *split_kernel_s(int n)
{
    switch (n) {
    case 1: return reinterpret_cast<const void *>(&fa::k_split_reduce<1, kS>);
    case 2: return reinterpret_cast<const void *>(&fa::k_split_reduce<2, kS>);
    case 3: return reinterpret_cast<const void *>(&fa::k_split_reduce<3, kS>);
    case 4: return reinterpret_cast<const void *>(&fa::k_split_reduce<4, kS>);
    case 5: return reinterpret_cast<const void *>(&fa::k_split_reduce<5, kS>);
    case 6: return reinterpret_cast<const void *>(&fa::k_split_reduce<6, kS>);
    case 7: return reinterpret_cast<const void *>(&fa::k_split_reduce<7, kS>);
    case 8: return reinterpret_cast<const void *>(&fa::k_split_reduce<8, kS>);
    default: return nullptr;
    }
}

// Slices per row of the split-row call: `splits` if given, else one slice per kSplitPacks packs.
// Each slice takes one pack per thread, so a slice holds at most kMaxBlock packs.
constexpr int kSplitPacks = 256;
constexpr int kMaxSplits = 64;

int split_geometry(int hidden, int splits, int *resolved, int *slice_packs, int *threads)
{
    const int packs = hidden / kPackElems;
    int s = splits != 0 ? splits : (packs + kSplitPacks - 1) / kSplitPacks;
    if (s < 1 || s > kMaxSplits)
        return FUSED_AR_ERR_INVALID;
    if (s > packs)
        s = packs;  // no empty slices
    const int sp = (packs + s - 1) / s;
    if (sp > kMaxBlock)
        return FUSED_AR_ERR_SHAPE;  // too few slices for one pack per thread
    *resolved = s;
    *slice_packs = sp;
    *threads = (sp + 63) / 64 * 64;
    return FUSED_AR_OK;
}

struct Step {
    const void *kernel;
    const char *name;
    unsigned grid, block, per_thread, launches;
    int n;             // inputs this step reads
    bool stream;       // non-temporal loads
    unsigned lds = 0;  // dynamic LDS reserved per workgroup (bytes), to cap workgroups per CU
};


struct Plan {
    int path;  // FUSED_AR_PATH_ONESTAGE, FUSED_AR_PATH_TWOSTAGE or kPathUnfusedPlan
    int steps;
    Step step[3];
    int chunk_rows;  // two-stage path: rows per chunk (m: one chunk)
    bool pipelined;  // two-stage path in chunks: stage 2 of a chunk and stage 1 of the next share
                     // a launch (k_pipe)
    bool stage1_residual;  // two-stage path with the residual add in stage 1
};

// Where the two-stage path adds the residual. In stage 1 unless the caller asks for the pages'
// split, or for a form that exists only with it (the LDS-staged stage 1, chunks of rows): then
// stage 1 stores the reduced rows into `out` and stage 2 reads them back and adds the residual.
// Measured on MI355X (HBM-cold, bit-identical results): n = 4, m = 4096, hidden 7168 89.2 ->
// 80.7 us; n = 8, 8192 x 8192 289.1 -> 272.9 us; n = 8, m = 4096, hidden 7168 131.5 -> 124.0 us:
// one plane less read and one less written.
bool residual_in_stage1(const Options &o)
{
    if (o.residual_stage != FUSED_AR_RESIDUAL_AUTO)
        return o.residual_stage == FUSED_AR_RESIDUAL_STAGE1;
    return !o.lds_stage1 && o.stage_rows <= 0;
}

// Rows per chunk of the two-stage path, and whether the chunks are pipelined.
int chunk_rows_for(const Options &o, int m)
{
    if (o.stage_rows == -1)
        return m;
    if (o.stage_rows > 0)
        return o.stage_rows < m ? o.stage_rows : m;
    return m;
}

bool pipelined_for(const Options &o)
{
    return o.schedule == FUSED_AR_CHUNKS_PIPELINED;
}

size_t flat_launches(size_t packs)
{
    return (packs + kFlatPacksPerLaunch - 1) / kFlatPacksPerLaunch;
}

// A flat kernel over total_packs packs, one per thread, in launches of at most
// kFlatPacksPerLaunch packs; `grid` is that of the first launch.
Step flat_step(const void *kernel, const char *name, int n, size_t total_packs, unsigned block,
               bool stream)
{
    const size_t first = total_packs < kFlatPacksPerLaunch ? total_packs : kFlatPacksPerLaunch;
    const size_t launches = (total_packs + kFlatPacksPerLaunch - 1) / kFlatPacksPerLaunch;
    return {kernel, name, static_cast<unsigned>((first + block - 1) / block), block, 1,
            static_cast<unsigned>(launches), n, stream};
}

// The launches of one call along `path` (one-stage, two-stage or the unfused sequence).
int make_plan(int n, int m, int hidden, int path, const Options &o, Plan *plan)
{
    memset(plan, 0, sizeof(*plan));
    plan->path = path;
    if (m == 0)
        return FUSED_AR_OK;
    const int packs = hidden / kPackElems;
    const bool stream = use_stream(o, n, m, hidden);
    const bool capped = rows_capped(stream, m);
    int ppt, threads;
    const int rc = row_geometry(packs, m, o.ppt, capped, &ppt, &threads);
    if (rc != FUSED_AR_OK)
        return rc;
    const size_t total = (size_t)m * (size_t)packs;
    const int64_t launches = ((int64_t)m + kRowsPerLaunch - 1) / kRowsPerLaunch;
    Step rows{nullptr, "", static_cast<unsigned>(m < kRowsPerLaunch ? m : kRowsPerLaunch),
              static_cast<unsigned>(threads), static_cast<unsigned>(ppt),
              static_cast<unsigned>(launches), n, stream};
    if (capped)
        rows.lds = kRowCapLds;
    if (path == FUSED_AR_PATH_ONESTAGE) {
        rows.kernel = row_kernel(n, ppt, o.bpermute, true, stream);
        rows.name = "onestage";
        plan->steps = 1;
        plan->step[0] = rows;
        return FUSED_AR_OK;
    }
    if (o.lds_stage1) {
        plan->step[0] = flat_step(lds_kernel(n, stream), "stage1_reduce_lds", n, total,
                                  64u * static_cast<unsigned>(n), stream);
    } else {
        plan->step[0] = flat_step(flat_kernel(n, stream), "stage1_reduce", n, total,
                                  flat_block_for(o, total), stream);
    }
    rows.n = 1;
    if (path == FUSED_AR_PATH_TWOSTAGE && residual_in_stage1(o)) {
        // stage 1 writes residual_out; stage 2 is the plain RMSNorm of it
        plan->stage1_residual = true;
        plan->chunk_rows = m;
        plan->step[0] = flat_step(flat_residual_kernel(n, stream), "stage1_reduce_residual", n,
                                  total, flat_block_for(o, total), stream);
        rows.kernel = row_kernel(1, ppt, o.bpermute, false, stream);
        rows.name = "stage2_rmsnorm";
        plan->steps = 2;
        plan->step[1] = rows;
        return FUSED_AR_OK;
    }
    if (path == FUSED_AR_PATH_TWOSTAGE) {
        rows.kernel = row_kernel(1, ppt, o.bpermute, true, stream);
        rows.name = "stage2_norm";
        const int r = chunk_rows_for(o, m);
        plan->chunk_rows = r;
        plan->steps = 2;
        if (r == m) {
            plan->step[1] = rows;
            return FUSED_AR_OK;
        }
        // chunks of r <= kRowsPerLaunch rows: one row launch per chunk
        const int64_t chunks = ((int64_t)m + r - 1) / r;
        const int last = static_cast<int>(m - (chunks - 1) * r);
        const size_t chunk_packs = (size_t)r * (size_t)packs;
        const size_t last_packs = (size_t)last * (size_t)packs;
        if (o.lds_stage1)
            plan->step[0] = flat_step(lds_kernel(n, stream), "stage1_reduce_lds", n, chunk_packs,
                                      64u * static_cast<unsigned>(n), stream);
        else
            plan->step[0] = flat_step(flat_kernel(n, stream), "stage1_reduce", n, chunk_packs,
                                      flat_block_for(o, chunk_packs), stream);
        rows.grid = static_cast<unsigned>(r);
        if (!pipelined_for(o)) {
            // stage 1 then stage 2 on each chunk in turn
            plan->step[0].launches = static_cast<unsigned>(
                (size_t)(chunks - 1) * flat_launches(chunk_packs) + flat_launches(last_packs));
            rows.launches = static_cast<unsigned>(chunks);
            plan->step[1] = rows;
            return FUSED_AR_OK;
        }
        // stage 1 of the first chunk; chunks - 1 launches of stage 2 of chunk c with stage 1 of
        // chunk c + 1; stage 2 of the last chunk
        plan->pipelined = true;
        plan->step[0].launches = static_cast<unsigned>(flat_launches(chunk_packs));
        Step pipe = rows;
        pipe.kernel = pipe_kernel(n, ppt, stream);
        pipe.name = "stage_pipe";
        pipe.n = n;
        pipe.grid = static_cast<unsigned>(r + (chunks == 2 ? last : r));
        pipe.launches = static_cast<unsigned>(chunks - 1);
        plan->step[1] = pipe;
        rows.grid = static_cast<unsigned>(last);
        rows.launches = 1;
        plan->step[2] = rows;
        plan->steps = 3;
        return FUSED_AR_OK;
    }
    // unfused: the residual add is the flat reduce of (reduced, residual); then a plain RMSNorm
    plan->step[1] = flat_step(flat_kernel(2, stream), "residual_add", 2, total,
                              flat_block_for(o, total), stream);
    rows.kernel = row_kernel(1, ppt, o.bpermute, false, stream);
    rows.name = "rmsnorm";
    plan->steps = 3;
    plan->step[2] = rows;
    return FUSED_AR_OK;
}

int launch(const void *kernel, unsigned grid, unsigned block, void *args, hipStream_t stream,
           unsigned lds = 0)
{
    void *params[] = {args};
    const hipError_t e = hipLaunchKernel(kernel, dim3(grid), dim3(block), params, lds, stream);
    return e == hipSuccess ? FUSED_AR_OK : static_cast<int>(e);
}

// One workgroup per row, at most kRowsPerLaunch rows per launch; later launches start
// kRowsPerLaunch rows further into every [m, hidden] buffer.
int run_rows(const Step &s, const RowArgs &args, int m, int packs, hipStream_t stream)
{
    for (int64_t first = 0; first < m; first += kRowsPerLaunch) {
        const int rows = static_cast<int>(m - first < kRowsPerLaunch ? m - first : kRowsPerLaunch);
        const size_t skip = (size_t)first * (size_t)packs;  // in packs
        RowArgs a = args;
        for (int i = 0; i < s.n; ++i)
            a.in[i] += skip;
        a.residual += skip;
        a.residual_out += skip;
        a.out += skip;
        const int rc = launch(s.kernel, static_cast<unsigned>(rows), s.block, &a, stream, s.lds);
        if (rc != FUSED_AR_OK)
            return rc;
    }
    return FUSED_AR_OK;
}

// At most kFlatPacksPerLaunch packs per launch; later launches start that many packs further into
// every buffer.
int run_flat(const Step &s, const u32x4 *const *inputs, size_t total_packs, u32x4 *dst,
             hipStream_t stream)
{
    for (size_t first = 0; first < total_packs; first += kFlatPacksPerLaunch) {
        const size_t left = total_packs - first;
        FlatArgs a{};
        for (int i = 0; i < s.n; ++i)
            a.in[i] = inputs[i] + first;
        a.out = dst + first;
        a.packs = static_cast<uint32_t>(left < kFlatPacksPerLaunch ? left : kFlatPacksPerLaunch);
        const unsigned grid = (a.packs + s.block - 1) / s.block;
        const int rc = launch(s.kernel, grid, s.block, &a, stream);
        if (rc != FUSED_AR_OK)
            return rc;
    }
    return FUSED_AR_OK;
}

// The two-stage path in chunks of plan.chunk_rows rows (fewer than m). `a` holds the call's
// buffers at row 0; each chunk's stage 1 writes its reduced rows into `out`, and its stage 2 reads
// them back and overwrites them with the normalised rows. Sequential: stage 1 and stage 2 of each
// chunk in turn. Pipelined: stage 1 of the first chunk, then launches of stage 2 of chunk c
// together with stage 1 of chunk c + 1, then stage 2 of the last chunk.
int run_chunks(const Plan &plan, const u32x4 *const *ins, int n, const RowArgs &a, int m,
               int packs, hipStream_t stream)
{
    const int64_t r = plan.chunk_rows;
    // the call's buffers moved to row `first`, stage 2 reading the reduced rows from `out`
    auto at_row = [&](int64_t first) {
        const size_t skip = (size_t)first * (size_t)packs;
        RowArgs c = a;
        c.in[0] = a.out + skip;
        for (int i = 1; i < fa::kMaxInputs; ++i)
            c.in[i] = nullptr;
        c.residual += skip;
        c.residual_out += skip;
        c.out += skip;
        return c;
    };
    auto stage1 = [&](int64_t first, int64_t rows) {
        const size_t skip = (size_t)first * (size_t)packs;
        const u32x4 *chunk_in[FUSED_AR_MAX_INPUTS];
        for (int i = 0; i < n; ++i)
            chunk_in[i] = ins[i] + skip;
        return run_flat(plan.step[0], chunk_in, (size_t)rows * (size_t)packs, a.out + skip,
                        stream);
    };
    const Step &norm = plan.pipelined ? plan.step[2] : plan.step[1];
    auto stage2 = [&](int64_t first, int64_t rows) {
        RowArgs c = at_row(first);
        return launch(norm.kernel, static_cast<unsigned>(rows), norm.block, &c, stream, norm.lds);
    };
    if (!plan.pipelined) {
        for (int64_t first = 0; first < m; first += r) {
            const int64_t rows = m - first < r ? m - first : r;
            int rc = stage1(first, rows);
            if (rc == FUSED_AR_OK)
                rc = stage2(first, rows);
            if (rc != FUSED_AR_OK)
                return rc;
        }
        return FUSED_AR_OK;
    }
    int rc = stage1(0, r);
    if (rc != FUSED_AR_OK)
        return rc;
    const Step &pipe = plan.step[1];
    int64_t first = 0;  // the chunk whose stage 2 is next
    for (; first + r < m; first += r) {
        const int64_t next = first + r;
        const int64_t next_rows = m - next < r ? m - next : r;
        fa::PipeArgs p{};
        p.norm = at_row(first);
        const size_t skip = (size_t)next * (size_t)packs;
        for (int i = 0; i < n; ++i)
            p.reduce.in[i] = ins[i] + skip;
        p.reduce.out = a.out + skip;
        p.reduce.packs = static_cast<uint32_t>(packs);
        p.norm_rows = static_cast<uint32_t>(r);
        rc = launch(pipe.kernel, static_cast<unsigned>(r + next_rows), pipe.block, &p, stream,
                    pipe.lds);
        if (rc != FUSED_AR_OK)
            return rc;
    }
    return stage2(first, m - first);
}

// The residual-adding stage 1 (k_flat_residual) over total_packs packs, in launches of at most
// kFlatPacksPerLaunch packs as run_flat.
int run_flat_residual(const Step &s, const u32x4 *const *inputs, const u32x4 *residual,
                      size_t total_packs, u32x4 *residual_out, hipStream_t stream)
{
    for (size_t first = 0; first < total_packs; first += kFlatPacksPerLaunch) {
        const size_t left = total_packs - first;
        fa::FlatResidualArgs a{};
        for (int i = 0; i < s.n; ++i)
            a.f.in[i] = inputs[i] + first;
        a.f.out = residual_out + first;
        a.f.packs = static_cast<uint32_t>(left < kFlatPacksPerLaunch ? left : kFlatPacksPerLaunch);
        a.residual = residual + first;
        const unsigned grid = (a.f.packs + s.block - 1) / s.block;
        const int rc = launch(s.kernel, grid, s.block, &a, stream);
        if (rc != FUSED_AR_OK)
            return rc;
    }
    return FUSED_AR_OK;
}

// Runs a validated call (m > 0) along `plan`.
int execute(const Plan &plan, const fa_bf16 *const *inputs, int n, const fa_bf16 *residual,
            const fa_bf16 *weight, float eps, int m, int hidden, fa_bf16 *residual_out,
            fa_bf16 *out, hipStream_t stream)
{
    const int packs = hidden / kPackElems;
    const size_t total = (size_t)m * (size_t)packs;
    const u32x4 *ins[FUSED_AR_MAX_INPUTS];
    for (int i = 0; i < n; ++i)
        ins[i] = reinterpret_cast<const u32x4 *>(inputs[i]);
    u32x4 *ro = reinterpret_cast<u32x4 *>(residual_out);
    u32x4 *o = reinterpret_cast<u32x4 *>(out);

    RowArgs a{};
    a.residual = reinterpret_cast<const u32x4 *>(residual);
    a.weight = reinterpret_cast<const u32x4 *>(weight);
    a.residual_out = ro;
    a.out = o;
    a.eps = eps;
    a.inv_hidden = static_cast<float>(1.0 / hidden);
    a.packs = packs;
    a.tiny_eps = eps < 0x1p-126f;

    if (plan.path == FUSED_AR_PATH_ONESTAGE) {
        for (int i = 0; i < n; ++i)
            a.in[i] = ins[i];
        return run_rows(plan.step[0], a, m, packs, stream);
    }
    if (plan.path == FUSED_AR_PATH_TWOSTAGE && plan.chunk_rows < m)
        return run_chunks(plan, ins, n, a, m, packs, stream);
    if (plan.path == FUSED_AR_PATH_TWOSTAGE && plan.stage1_residual) {
        int rc = run_flat_residual(plan.step[0], ins, a.residual, total, ro, stream);
        if (rc != FUSED_AR_OK)
            return rc;
        a.in[0] = ro;  // the plain RMSNorm of residual_out
        return run_rows(plan.step[1], a, m, packs, stream);
    }
    // Two-stage and unfused: the reduce writes the reduced rows into `out`.
    int rc = run_flat(plan.step[0], ins, total, o, stream);
    if (rc != FUSED_AR_OK)
        return rc;
    if (plan.path == FUSED_AR_PATH_TWOSTAGE) {
        // the row kernel with a single input reads the reduced rows back from `out` and
        // overwrites them with the normalised rows
        a.in[0] = o;
        return run_rows(plan.step[1], a, m, packs, stream);
    }
    // Unfused: residual_out = bf16(reduced + residual), then out = RMSNorm(residual_out).
    const u32x4 *pair[2] = {o, reinterpret_cast<const u32x4 *>(residual)};
    rc = run_flat(plan.step[1], pair, total, ro, stream);
    if (rc != FUSED_AR_OK)
        return rc;
    a.in[0] = ro;
    return run_rows(plan.step[2], a, m, packs, stream);
}

// The two kernels of the split-row form over a validated call (m > 0), the slice square-sums in
// `partial` (m * s floats of device memory).
int run_split(const fa_bf16 *const *inputs, int n, const fa_bf16 *residual, const fa_bf16 *weight,
              float eps, int m, int hidden, fa_bf16 *residual_out, fa_bf16 *out, int s,
              int slice_packs, int threads, float *partial, hipStream_t stream)
{
    const int packs = hidden / kPackElems;
    const bool stream_loads = use_stream(kDefaultOptions, n, m, hidden);
    const void *reduce_kernel = stream_loads ? split_kernel_s<true>(n) : split_kernel_s<false>(n);
    const void *norm_kernel = reinterpret_cast<const void *>(&fa::k_split_norm);
    // rows in launches of at most kRowsPerLaunch, as for the row kernels
    for (int64_t first = 0; first < m; first += kRowsPerLaunch) {
        const int rows = static_cast<int>(m - first < kRowsPerLaunch ? m - first : kRowsPerLaunch);
        const size_t skip = (size_t)first * (size_t)packs;  // in packs
        fa::SplitArgs a{};
        for (int i = 0; i < n; ++i)
            a.r.in[i] = reinterpret_cast<const u32x4 *>(inputs[i]) + skip;
        a.r.residual = reinterpret_cast<const u32x4 *>(residual) + skip;
        a.r.weight = reinterpret_cast<const u32x4 *>(weight);
        a.r.residual_out = reinterpret_cast<u32x4 *>(residual_out) + skip;
        a.r.out = reinterpret_cast<u32x4 *>(out) + skip;
        a.r.eps = eps;
        a.r.inv_hidden = static_cast<float>(1.0 / hidden);
        a.r.packs = packs;
        a.r.tiny_eps = eps < 0x1p-126f;
        a.partial = partial + (size_t)first * (size_t)s;
        a.splits = s;
        a.slice_packs = slice_packs;
        const unsigned grid = static_cast<unsigned>(rows) * static_cast<unsigned>(s);
        int rc = launch(reduce_kernel, grid, static_cast<unsigned>(threads), &a, stream);
        if (rc != FUSED_AR_OK)
            return rc;
        rc = launch(norm_kernel, grid, static_cast<unsigned>(threads), &a, stream);
        if (rc != FUSED_AR_OK)
            return rc;
    }
    return FUSED_AR_OK;
}

int resolve_path(int n, int m, int hidden, int path)
{
    if (path == FUSED_AR_PATH_UNFUSED)
        return kPathUnfusedPlan;
    return path == FUSED_AR_PATH_AUTO ? fused_ar_auto_path(n, m, hidden) : path;
}

}  // namespace

// Slice square-sums of fused_ar_rmsnorm_split_static: a fixed device array, so that the call needs
// no workspace and allocates nothing. Each GPU the library runs on holds its own copy until the
// process ends. In host code `scratch` names a host-side stand-in, not device memory: the copy on
// the current device is reached only through the address hipGetSymbolAddress returns for it, which
// static_scratch() looks up once per device and keeps.
static __device__ __align__(256) float scratch[FUSED_AR_STATIC_SCRATCH_FLOATS];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<float *> g_scratch[kMaxDevices];
std::mutex g_scratch_lookup;

// The device address of `scratch` on the current device: a HIP error code or FUSED_AR_OK.
int static_scratch(float **ptr)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return static_cast<int>(e);
    if (dev < 0 || dev >= kMaxDevices)
        return FUSED_AR_ERR_INVALID;
    float *p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> guard(g_scratch_lookup);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            void *q = nullptr;
            e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
            if (e != hipSuccess)
                return static_cast<int>(e);
            p = static_cast<float *>(q);
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return FUSED_AR_OK;
}

}  // namespace

// The automatic path on one GPU, from a sweep of both paths over n = 2..8, hidden = 2880..32768
// and m = 1..8192 (MI355X, graphs of calls for cache-sized problems, HBM-cold loops above): the
// one-stage path is faster or level everywhere (by up to 2.3x) except where a few rows are each
// too long for one CU. There the two-stage path's flat stage 1 spreads the reads over every CU:
// with rows that read (n inputs and the residual) at least 336 KiB it wins up to 16 rows, from
// 432 KiB up to 40 rows and from 512 KiB up to 48 rows (by up to 24 %; e.g. n = 8,
// hidden = 32768, m = 1: 5.8 against 7.7 us). The thresholds of the pages (fused_ar_auto_path_tp) weigh the link traffic
// between GPUs, which one GPU does not have.
struct TwoStageTier {
    uint64_t row_bytes;  // rows reading at least this many bytes...
    int max_m;           // ...take the two-stage path up to this many rows
};
constexpr TwoStageTier kTwoStageTiers[] = {{512u * 1024u, 48}, {432u * 1024u, 40}, {336u * 1024u, 16}};

extern "C" int fused_ar_auto_path(int n, int m, int hidden)
{
    if (n < 1 || n > FUSED_AR_MAX_INPUTS || m < 0 || hidden <= 0)
        return FUSED_AR_ERR_INVALID;
    const uint64_t row_read = 2ull * (uint64_t)(n + 1) * (uint64_t)hidden;
    for (const TwoStageTier &t : kTwoStageTiers)
        if (row_read >= t.row_bytes)
            return m <= t.max_m ? FUSED_AR_PATH_TWOSTAGE : FUSED_AR_PATH_ONESTAGE;
    return FUSED_AR_PATH_ONESTAGE;
}

extern "C" int fused_ar_auto_path_tp(int n, int m, int hidden)
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
    const int rc = check_scalars(n, m, hidden, eps, path, true);
    if (rc != FUSED_AR_OK || m == 0)
        return rc;
    return check_buffers(inputs, n, residual, weight, m, hidden, residual_out, out);
}

extern "C" int fused_ar_rmsnorm_ex(const fa_bf16 *const *inputs, int n, const fa_bf16 *residual,
                                   const fa_bf16 *weight, float eps, int m, int hidden,
                                   fa_bf16 *residual_out, fa_bf16 *out, int path,
                                   const fused_ar_options *options, hipStream_t stream)
{
    Options o;
    int rc = read_options(options, &o);
    if (rc != FUSED_AR_OK)
        return rc;
    const bool unfused = path == FUSED_AR_PATH_UNFUSED;
    rc = fused_ar_rmsnorm_check(inputs, n, residual, weight, eps, m, hidden, residual_out, out,
                                unfused ? FUSED_AR_PATH_AUTO : path);
    if (rc != FUSED_AR_OK || m == 0)
        return rc;
    Plan plan;
    rc = make_plan(n, m, hidden, resolve_path(n, m, hidden, path), o, &plan);
    if (rc != FUSED_AR_OK)
        return rc;
    return execute(plan, inputs, n, residual, weight, eps, m, hidden, residual_out, out, stream);
}

extern "C" int fused_ar_rmsnorm(const fa_bf16 *const *inputs, int n, const fa_bf16 *residual,
                                const fa_bf16 *weight, float eps, int m, int hidden,
                                fa_bf16 *residual_out, fa_bf16 *out, int path, hipStream_t stream)
{
    if (path == FUSED_AR_PATH_UNFUSED)
        return FUSED_AR_ERR_INVALID;  // the unfused sequence has its own entry point
    return fused_ar_rmsnorm_ex(inputs, n, residual, weight, eps, m, hidden, residual_out, out,
                               path, nullptr, stream);
}

extern "C" int fused_ar_unfused_rmsnorm(const fa_bf16 *const *inputs, int n,
                                        const fa_bf16 *residual, const fa_bf16 *weight, float eps,
                                        int m, int hidden, fa_bf16 *residual_out, fa_bf16 *out,
                                        hipStream_t stream)
{
    return fused_ar_rmsnorm_ex(inputs, n, residual, weight, eps, m, hidden, residual_out, out,
                               FUSED_AR_PATH_UNFUSED, nullptr, stream);
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
    const size_t plane = total_packs * sizeof(u32x4);
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
    const u32x4 *ins[FUSED_AR_MAX_INPUTS];
    for (int i = 0; i < n; ++i)
        ins[i] = reinterpret_cast<const u32x4 *>(inputs[i]);
    const bool nt = use_stream(kDefaultOptions, n - 1, m, hidden);  // reads n planes, no residual
    const Step s = flat_step(flat_kernel(n, nt), "stage1_reduce", n, total_packs,
                             flat_block_for(kDefaultOptions, total_packs), nt);
    return run_flat(s, ins, total_packs, reinterpret_cast<u32x4 *>(reduced), stream);
}

extern "C" size_t fused_ar_split_workspace_bytes(int m, int hidden, int splits)
{
    if (m < 0 || hidden <= 0 || hidden % kPackElems != 0 || hidden > FUSED_AR_MAX_HIDDEN)
        return 0;
    int s, sp, threads;
    if (split_geometry(hidden, splits, &s, &sp, &threads) != FUSED_AR_OK)
        return 0;
    return (size_t)m * (size_t)s * sizeof(float);
}

extern "C" int fused_ar_rmsnorm_split(const fa_bf16 *const *inputs, int n, const fa_bf16 *residual,
                                      const fa_bf16 *weight, float eps, int m, int hidden,
                                      fa_bf16 *residual_out, fa_bf16 *out, int splits,
                                      void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    int rc = check_scalars(n, m, hidden, eps, FUSED_AR_PATH_ONESTAGE, true);
    if (rc != FUSED_AR_OK)
        return rc;
    int s, slice_packs, threads;
    rc = split_geometry(hidden, splits, &s, &slice_packs, &threads);
    if (rc != FUSED_AR_OK || m == 0)
        return rc;
    rc = check_buffers(inputs, n, residual, weight, m, hidden, residual_out, out);
    if (rc != FUSED_AR_OK)
        return rc;
    const size_t need = (size_t)m * (size_t)s * sizeof(float);
    Span ws;
    if (workspace == nullptr || workspace_bytes < need || !make_span(workspace, need, &ws))
        return FUSED_AR_ERR_INVALID;
    if (!aligned16(workspace))
        return FUSED_AR_ERR_ALIGN;
    const size_t plane = (size_t)m * (size_t)hidden * sizeof(fa_bf16);
    Span other;
    for (int i = 0; i < n; ++i)
        if (make_span(inputs[i], plane, &other) && overlaps(ws, other))
            return FUSED_AR_ERR_ALIAS;
    const void *bufs[3] = {residual, residual_out, out};
    for (const void *b : bufs)
        if (make_span(b, plane, &other) && overlaps(ws, other))
            return FUSED_AR_ERR_ALIAS;
    if (make_span(weight, (size_t)hidden * sizeof(fa_bf16), &other) && overlaps(ws, other))
        return FUSED_AR_ERR_ALIAS;

    return run_split(inputs, n, residual, weight, eps, m, hidden, residual_out, out, s, slice_packs,
                     threads, static_cast<float *>(workspace), stream);
}

extern "C" int fused_ar_rmsnorm_split_static(const fa_bf16 *const *inputs, int n,
                                             const fa_bf16 *residual, const fa_bf16 *weight,
                                             float eps, int m, int hidden, fa_bf16 *residual_out,
                                             fa_bf16 *out, int splits, hipStream_t stream)
{
    int rc = check_scalars(n, m, hidden, eps, FUSED_AR_PATH_ONESTAGE, true);
    if (rc != FUSED_AR_OK)
        return rc;
    int s, slice_packs, threads;
    rc = split_geometry(hidden, splits, &s, &slice_packs, &threads);
    if (rc != FUSED_AR_OK || m == 0)
        return rc;
    rc = check_buffers(inputs, n, residual, weight, m, hidden, residual_out, out);
    if (rc != FUSED_AR_OK)
        return rc;
    if ((uint64_t)m * (uint64_t)s > (uint64_t)FUSED_AR_STATIC_SCRATCH_FLOATS)
        return FUSED_AR_ERR_SCRATCH;
    float *partial = nullptr;
    rc = static_scratch(&partial);
    if (rc != FUSED_AR_OK)
        return rc;
    return run_split(inputs, n, residual, weight, eps, m, hidden, residual_out, out, s, slice_packs,
                     threads, partial, stream);
}

extern "C" int fused_ar_describe_launch_ex(int n, int m, int hidden, int path,
                                           const fused_ar_options *options,
                                           fused_ar_launch_plan *plan)
{
    int rc = check_scalars(n, m, hidden, 0.0f,
                           path == FUSED_AR_PATH_UNFUSED ? FUSED_AR_PATH_AUTO : path, true);
    if (rc != FUSED_AR_OK)
        return rc;
    if (plan == nullptr)
        return FUSED_AR_ERR_INVALID;
    Options o;
    rc = read_options(options, &o);
    if (rc != FUSED_AR_OK)
        return rc;
    Plan p;
    rc = make_plan(n, m, hidden, resolve_path(n, m, hidden, path), o, &p);
    if (rc != FUSED_AR_OK)
        return rc;
    memset(plan, 0, sizeof(*plan));
    plan->path = path == FUSED_AR_PATH_UNFUSED ? FUSED_AR_PATH_UNFUSED : p.path;
    plan->kernels = p.steps;
    for (int i = 0; i < p.steps; ++i) {
        fused_ar_kernel_launch &k = plan->launch[i];
        strncpy(k.name, p.step[i].name, sizeof(k.name) - 1);
        k.grid = p.step[i].grid;
        k.block = p.step[i].block;
        k.per_thread = p.step[i].per_thread;
        k.launches = p.step[i].launches;
        k.streaming = p.step[i].stream ? 1u : 0u;
        k.lds_bytes = p.step[i].lds;
    }
    return FUSED_AR_OK;
}

extern "C" int fused_ar_describe_launch(int n, int m, int hidden, int path,
                                        fused_ar_launch_plan *plan)
{
    return fused_ar_describe_launch_ex(n, m, hidden, path, nullptr, plan);
}

extern "C" const char *fused_ar_strerror(int status)
{
    switch (status) {
    case FUSED_AR_OK: return "success";
    case FUSED_AR_ERR_INVALID: return "invalid argument (null pointer, n, m, hidden, eps, path or option out of range)";
    case FUSED_AR_ERR_SHAPE:
        return "unsupported shape (hidden must be a multiple of 8 and at most 32768, and a row, or a "
               "slice of a split row, must fit one 1024-thread workgroup at the packs per thread or "
               "slice count asked for)";
    case FUSED_AR_ERR_ALIGN: return "a device pointer is not 16-byte aligned";
    case FUSED_AR_ERR_ALIAS: return "forbidden overlap between output and other buffers";
    case FUSED_AR_ERR_SCRATCH:
        return "the call needs more slice square-sums (m * slices) than the library's static "
               "scratch holds (FUSED_AR_STATIC_SCRATCH_FLOATS)";
    default: break;
    }
    if (status > 0)
        return hipGetErrorString(static_cast<hipError_t>(status));
    return "unknown status";
}
