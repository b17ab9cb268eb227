// kernels.h - the gfx950 kernels of the fused all-reduce + residual + RMSNorm epilogue.
//
//   k_rows<N, PPT>     one workgroup per row: N-way reduce, residual add, square-sum, RMSNorm.
//                      With N inputs it is the one-stage path (aiter PR #3817, Technical Details >
//                      1stage); with N = 1 reading the reduced rows it is stage 2 of the two-stage
//                      path (Technical Details > 2stage > stage-2 RMSNorm reduce).
//   k_flat_reduce<N>   stage 1 of the two-stage path in the pages' split, and the reduce alone:
//                      one thread per pack, N-way fp32 reduce, one bf16 store, no LDS and no
//                      workgroup barrier (Technical Details > 2stage > reduce-scatter).
//   k_split_reduce<N>, k_split_norm
//                      split rows: the one-stage result with each row cut into slices on separate
//                      workgroups, the second kernel combining the slices' square-sums.
//   k_flat_residual<N> stage 1 with the residual add moved into it (writes residual_out): the
//                      two-stage path's default first kernel.
//   k_pipe<N, PPT>     the two-stage path in row chunks: stage 2 of one chunk and stage 1 of the
//                      next in one launch.
//   k_stage1_lds<N>    the LDS-staged, one-wave-per-input stage 1 that the flat reduce replaced,
//                      kept for comparison.
//
// All read and write 16-byte packs of eight bf16; a row of `hidden` elements is hidden / 8 packs
// and consecutive lanes touch consecutive packs, so every wave access is 1 KiB contiguous.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "bf16x8.h"
#include "wave_sum.h"

namespace fa {

constexpr int kMaxInputs = 8;
constexpr int kMaxWaves = 16;  // 1024 threads

struct RowArgs {
    const u32x4 *in[kMaxInputs];  // N partial sums, [m, packs] packs each
    const u32x4 *residual;        // [m, packs]
    const u32x4 *weight;          // [packs]
    u32x4 *residual_out;          // [m, packs]; may equal residual
    u32x4 *out;                   // [m, packs]; may equal in[0] when N == 1 (stage 2)
    float eps;
    float inv_hidden;             // 1 / hidden rounded to fp32: the mean is the square-sum times it
    int packs;                    // packs per row = hidden / 8
    int tiny_eps;                 // eps < 2^-126: mean + eps may be subnormal (see rsqrt_f32)
};

struct FlatArgs {
    const u32x4 *in[kMaxInputs];
    u32x4 *out;
    uint32_t packs;  // packs in this launch (the host splits larger problems into launches)
};

// Sum of the N packs in input order, in fp32, starting from input 0.
template <int N>
__device__ __forceinline__ F8 reduce_packs(const u32x4 (&x)[N])
{
    F8 acc = widen(x[0]);
#pragma unroll
    for (int i = 1; i < N; ++i)
        add_into(acc, widen(x[i]));
    return acc;
}

// Per-pack arithmetic of the split-row kernels. k_rows spells the same steps out inline: moving
// them into these helpers changes the compiler's instruction order there, measured 1.5 % slower
// on the one-row (decode) case.

// residual_out of one pack: the N-way sum rounded to bf16, plus the residual, rounded to bf16.
template <int N>
__device__ __forceinline__ u32x4 add_residual(const u32x4 (&x)[N], u32x4 res)
{
    F8 sum = widen(narrow(reduce_packs<N>(x)));  // the reduced value, in bf16
    add_into(sum, widen(res));
    return narrow(sum);
}

// ss plus the squares of a pack's eight values (each x * x is exact in fp32).
__device__ __forceinline__ float add_squares(const F8 &y, float ss)
{
#pragma unroll
    for (int e = 0; e < 8; ++e)
        ss = __builtin_fmaf(y.v[e], y.v[e], ss);
    return ss;
}

// out of one pack: (x * rstd) * weight in fp32, rounded to bf16.
__device__ __forceinline__ u32x4 normalise(const F8 &y, const F8 &g, float rstd)
{
    F8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e)
        o.v[e] = (y.v[e] * rstd) * g.v[e];
    return narrow(o);
}

// Below this fp32 square-sum a row's squares may have lost bits to the subnormal range (each
// y * y under 2^-126 is rounded to a multiple of 2^-149), enough to move `out` past its 1-ulp band:
// with eps below the normal range the row kernel then sums the squares again at a 2^100 scale.
// Above it those roundings add at most hidden * 2^-150 < 2^-135, under 2^-25 of the sum.
constexpr float kTinySquareSum = 0x1p-110f;

// 1 / sqrt(v) for v = mean + eps >= eps by the hardware reciprocal square root (v_rsq_f32, within
// 1 ulp in fp32). Below the normal range v is scaled by 2^24 first (and the result by 2^12), so
// subnormal arguments keep the same accuracy; 0 gives +inf. They are possible only when eps itself
// is below the normal range (eps = 0 or subnormal), which the host flags: otherwise the scaling is
// left out of the row's path (a uniform branch).
__device__ __forceinline__ float rsqrt_f32(float v, int tiny_eps)
{
    if (!tiny_eps)
        return __builtin_amdgcn_rsqf(v);
    const bool tiny = v < 0x1p-126f;
    const float r = __builtin_amdgcn_rsqf(tiny ? v * 0x1p24f : v);
    return tiny ? 0x1p12f * r : r;
}

// Asks for kernel arguments in scalar registers at this point, in one statement. Placed at the top
// of a kernel with every pointer the kernel dereferences and the sizes that decide its branches, it
// makes the compiler issue all of the argument loads together and wait for them once; left to
// itself, it loads the pointers used inside a branch only after waiting for the values that decide
// the branch, a second dependent round trip before the first data load (measured: 2-3 % of a
// decode-sized call). All kMaxInputs input pointers are named, used or not: they come in the same
// argument block. The split-row kernels do without: there it measured slower (their combine reads
// no input pointers and waits on the slice partials anyway).
__device__ __forceinline__ void args_in_sgprs(const u32x4 *const (&in)[kMaxInputs], const void *p0,
                                              uint32_t u0, uint32_t u1)
{
    asm volatile("" ::"s"(in[0]), "s"(in[1]), "s"(in[2]), "s"(in[3]), "s"(in[4]), "s"(in[5]),
                 "s"(in[6]), "s"(in[7]), "s"(p0), "s"(u0), "s"(u1));
}

// The same for the row kernel, which also keeps the row statistic's arguments: named as outputs
// of the statement they count as values it produced, so the compiler holds them in registers
// instead of loading them from the argument block again after the barrier.
__device__ __forceinline__ void args_in_sgprs(const RowArgs &a, float &eps, float &inv_hidden,
                                              int &tiny_eps)
{
    asm volatile(""
                 : "+s"(eps), "+s"(inv_hidden), "+s"(tiny_eps)
                 : "s"(a.in[0]), "s"(a.in[1]), "s"(a.in[2]), "s"(a.in[3]), "s"(a.in[4]),
                   "s"(a.in[5]), "s"(a.in[6]), "s"(a.in[7]), "s"(a.residual), "s"(a.weight),
                   "s"(a.residual_out), "s"(a.out), "s"(a.packs), "s"(blockDim.x));
}

// A pack at a byte offset from a wave-uniform base (the base stays in scalar registers, the
// per-lane offset is 32 bits). load_pack is an ordinary load (the weight, read by every row, and
// inputs that may still be cached); load_stream is a non-temporal load (inputs streamed from HBM,
// so that they do not displace reused lines). store_stream is a non-temporal store for the
// outputs.
__device__ __forceinline__ u32x4 load_pack(const char *base, uint32_t off)
{
    return *reinterpret_cast<const u32x4 *>(base + off);
}

__device__ __forceinline__ u32x4 load_stream(const char *base, uint32_t off)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(base + off));
}

__device__ __forceinline__ void store_stream(char *base, uint32_t off, u32x4 v)
{
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(base + off));
}

__device__ __forceinline__ void store_pack(char *base, uint32_t off, u32x4 v)
{
    *reinterpret_cast<u32x4 *>(base + off) = v;
}

// The load of a pack that is read once: non-temporal when kStream (data arriving from HBM; the hint
// keeps it from displacing reused lines), an ordinary load otherwise (data that may still be in
// the L2 or the Infinity Cache, where an ordinary load finds it).
template <bool kStream>
__device__ __forceinline__ u32x4 load_once(const char *base, uint32_t off)
{
    if constexpr (kStream)
        return load_stream(base, off);
    else
        return load_pack(base, off);
}

// One row of the row kernel (k_rows: workgroup b handles row b; the host launches one workgroup
// per row, splitting very tall problems into several launches); thread t handles packs t,
// t + blockDim.x, ..., PPT of them. `eps`, `inv_hidden` and `tiny_eps` are the caller's copies of
// the argument fields (see args_in_sgprs). For each of its packs a thread loads the N inputs, the residual and the weight, reduces,
// writes residual_out and accumulates the square-sum, keeping only the bf16 residual_out and
// weight packs; one workgroup reduction then gives the row statistic and the normalised row is
// written from those registers.
//   kBpermute  wave reduction by the ds_bpermute butterfly instead of DPP (bit-identical; for
//              comparison with the design the pages replaced).
//   kResidual  false: a plain RMSNorm of in[0] (N == 1), with no residual and no residual_out;
//              the last kernel of the unfused sequence.
//   kStream    non-temporal loads of the inputs and the residual (see load_once); with N == 1 the
//              input is the reduced rows the flat reduce has just stored (two-stage path, unfused
//              sequence), which may still be in the Infinity Cache, so it is always loaded normally.
template <int N, int PPT, bool kBpermute, bool kResidual, bool kStream>
__device__ __forceinline__ void row_pass(const RowArgs &a, float eps, float inv_hidden,
                                         int tiny_eps, uint32_t row, float *slots)
{
    static_assert(kResidual || N == 1, "the plain RMSNorm reads one input");
    const uint32_t tid = threadIdx.x;
    const uint32_t nthreads = blockDim.x;
    const uint32_t packs = (uint32_t)a.packs;
    const size_t row_bytes = (size_t)row * packs * sizeof(u32x4);
    const char *weight = reinterpret_cast<const char *>(a.weight);
    const char *in[N];
#pragma unroll
    for (int i = 0; i < N; ++i)
        in[i] = reinterpret_cast<const char *>(a.in[i]) + row_bytes;
    const char *residual = reinterpret_cast<const char *>(a.residual) + row_bytes;
    char *residual_out = reinterpret_cast<char *>(a.residual_out) + row_bytes;
    char *out = reinterpret_cast<char *>(a.out) + row_bytes;

    u32x4 ro[PPT];
    u32x4 w[PPT];
    F8 y1;  // one pack per thread: residual_out widened once, kept for the normalisation
    float ss = 0.0f;
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
        const uint32_t p = tid + k * nthreads;
        if (p < packs) {
            const uint32_t off = p * (uint32_t)sizeof(u32x4);
            u32x4 x[N];
#pragma unroll
            for (int i = 0; i < N; ++i)
                x[i] = (N == 1) ? load_pack(in[i], off) : load_once<kStream>(in[i], off);
            u32x4 res;
            if constexpr (kResidual)
                res = load_once<kStream>(residual, off);
            w[k] = load_pack(weight, off);
            // all of this slot's loads are in flight before any arithmetic waits on one
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (kResidual) {
                F8 sum = widen(narrow(reduce_packs<N>(x)));  // the reduced value, in bf16
                add_into(sum, widen(res));
                ro[k] = narrow(sum);
                store_stream(residual_out, off, ro[k]);
            } else {
                ro[k] = x[0];
            }
            const F8 y = widen(ro[k]);
            if constexpr (PPT == 1)
                y1 = y;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                ss = __builtin_fmaf(y.v[e], y.v[e], ss);  // y * y is exact in fp32
        }
    }

    const float total = block_sum<kBpermute>(ss, slots);
    float rstd = rsqrt_f32(total * inv_hidden + eps, tiny_eps);
    if (tiny_eps && total < kTinySquareSum) {
        // eps = 0 or subnormal and a row so small that squares below 2^-126 lost bits or vanished:
        // the square-sum again over x * 2^100 (exact scaling, squares exact and normal), mean + eps
        // scaled by 2^200 likewise, and the reciprocal root scaled back by 2^100. A uniform branch
        // (tiny_eps and total are the same in every wave); the second sum has LDS of its own.
        __shared__ float slots_scaled[kMaxWaves];
        float ss2 = 0.0f;
#pragma unroll
        for (int k = 0; k < PPT; ++k) {
            if (tid + k * nthreads < packs) {
                const F8 y = PPT == 1 ? y1 : widen(ro[k]);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float z = y.v[e] * 0x1p100f;
                    ss2 = __builtin_fmaf(z, z, ss2);
                }
            }
        }
        const float total2 = block_sum<kBpermute>(ss2, slots_scaled);
        rstd = 0x1p100f * __builtin_amdgcn_rsqf(total2 * inv_hidden + eps * 0x1p100f * 0x1p100f);
    }

#pragma unroll
    for (int k = 0; k < PPT; ++k) {
        const uint32_t p = tid + k * nthreads;
        if (p < packs) {
            const uint32_t off = p * (uint32_t)sizeof(u32x4);
            // with more packs per thread, widening again costs fewer registers than keeping them
            const F8 y = PPT == 1 ? y1 : widen(ro[k]);
            const F8 g = widen(w[k]);
            F8 o;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                o.v[e] = (y.v[e] * rstd) * g.v[e];
            store_stream(out, off, narrow(o));
        }
    }
}

template <int N, int PPT, bool kBpermute, bool kResidual, bool kStream>
__global__ void __launch_bounds__(1024) k_rows(RowArgs a)
{
    __shared__ float slots[kMaxWaves];
    float eps = a.eps, inv_hidden = a.inv_hidden;
    int tiny_eps = a.tiny_eps;
    args_in_sgprs(a, eps, inv_hidden, tiny_eps);
    row_pass<N, PPT, kBpermute, kResidual, kStream>(a, eps, inv_hidden, tiny_eps, blockIdx.x,
                                                     slots);
}

// Flat N-way reduce: thread t of workgroup b handles pack b * blockDim.x + t (one pack per thread;
// the host launches enough workgroups, splitting more than 2^30 packs into several launches).
template <int N, bool kStream>
__global__ void __launch_bounds__(1024) k_flat_reduce(FlatArgs a)
{
    args_in_sgprs(a.in, a.out, a.packs, blockDim.x);
    const uint32_t first = blockIdx.x * blockDim.x;
    if (first + threadIdx.x >= a.packs)
        return;
    const size_t bytes = (size_t)first * sizeof(u32x4);
    const uint32_t off = threadIdx.x * (uint32_t)sizeof(u32x4);
    u32x4 x[N];
#pragma unroll
    for (int i = 0; i < N; ++i)
        x[i] = load_once<kStream>(reinterpret_cast<const char *>(a.in[i]) + bytes, off);
    __builtin_amdgcn_sched_barrier(0);  // all N loads in flight before the first add
    // the reduced rows are read straight back by the next kernel: an ordinary store, so that they
    // can stay in the Infinity Cache
    store_pack(reinterpret_cast<char *>(a.out) + bytes, off, narrow(reduce_packs<N>(x)));
}

// Stage 1 of the two-stage path with the residual add moved into it: one thread per pack reduces
// the N inputs, rounds to bf16, adds the residual and stores residual_out (the same per-pack
// arithmetic as the row kernel), so that stage 2 is a plain RMSNorm of residual_out and no
// scratch plane is written and read back. No LDS, no barrier. `out` of FlatArgs is residual_out;
// the residual may be residual_out itself (each thread reads its pack before writing it).
struct FlatResidualArgs {
    FlatArgs f;
    const u32x4 *residual;
};

template <int N, bool kStream>
__global__ void __launch_bounds__(1024) k_flat_residual(FlatResidualArgs a)
{
    asm volatile("" ::"s"(a.f.in[0]), "s"(a.f.in[1]), "s"(a.f.in[2]), "s"(a.f.in[3]),
                 "s"(a.f.in[4]), "s"(a.f.in[5]), "s"(a.f.in[6]), "s"(a.f.in[7]), "s"(a.residual),
                 "s"(a.f.out), "s"(a.f.packs), "s"(blockDim.x));
    const uint32_t first = blockIdx.x * blockDim.x;
    if (first + threadIdx.x >= a.f.packs)
        return;
    const size_t bytes = (size_t)first * sizeof(u32x4);
    const uint32_t off = threadIdx.x * (uint32_t)sizeof(u32x4);
    u32x4 x[N];
#pragma unroll
    for (int i = 0; i < N; ++i)
        x[i] = load_once<kStream>(reinterpret_cast<const char *>(a.f.in[i]) + bytes, off);
    const u32x4 res = load_once<kStream>(reinterpret_cast<const char *>(a.residual) + bytes, off);
    __builtin_amdgcn_sched_barrier(0);  // all N + 1 loads in flight before the first add
    // read straight back by the RMSNorm kernel: an ordinary store, so that it can stay cached
    store_pack(reinterpret_cast<char *>(a.f.out) + bytes, off, add_residual<N>(x, res));
}

// Two-stage path in row chunks, pipelined: one launch runs stage 2 on the rows of one chunk,
// whose reduced rows the previous launch stored into `out`, and stage 1 on the rows of the next
// chunk. The launch boundary orders the two stages of a chunk; within a launch the two kinds of
// workgroup touch disjoint rows. Workgroups [0, norm_rows) take stage 2 (the row kernel's pass
// with one input, the call's geometry, so `out` is bit-identical to the other paths); workgroups
// [norm_rows, norm_rows + reduce_rows) take stage 1 of one row each (thread t reduces packs
// t, t + blockDim.x, ... of the row, the same per-pack arithmetic as k_flat_reduce).
struct PipeArgs {
    RowArgs norm;     // stage 2: in[0] = the reduced rows of the chunk (in `out`), other buffers
                      // at the same chunk's first row
    FlatArgs reduce;  // stage 1: in[0..N-1] and out (the scratch) at the next chunk's first row;
                      // `packs` is the row length here
    uint32_t norm_rows;
};

// Stage 1 of one row: the N-way reduce of each of the thread's packs, stored into the scratch.
template <int N, int PPT, bool kStream>
__device__ __forceinline__ void reduce_row(const FlatArgs &f, uint32_t row)
{
    const uint32_t packs = f.packs;
    const size_t row_bytes = (size_t)row * packs * sizeof(u32x4);
    char *dst = reinterpret_cast<char *>(f.out) + row_bytes;
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
        const uint32_t p = threadIdx.x + k * blockDim.x;
        if (p < packs) {
            const uint32_t off = p * (uint32_t)sizeof(u32x4);
            u32x4 x[N];
#pragma unroll
            for (int i = 0; i < N; ++i)
                x[i] = load_once<kStream>(reinterpret_cast<const char *>(f.in[i]) + row_bytes, off);
            __builtin_amdgcn_sched_barrier(0);
            store_pack(dst, off, narrow(reduce_packs<N>(x)));
        }
    }
}

template <int N, int PPT, bool kStream>
__global__ void __launch_bounds__(1024) k_pipe(PipeArgs a)
{
    __shared__ float slots[kMaxWaves];
    if (blockIdx.x < a.norm_rows)
        row_pass<1, PPT, false, true, kStream>(a.norm, a.norm.eps, a.norm.inv_hidden,
                                               a.norm.tiny_eps, blockIdx.x, slots);
    else
        reduce_row<N, PPT, kStream>(a.reduce, blockIdx.x - a.norm_rows);
}

// Split rows: each row is cut into `splits` slices of slice_packs packs, one workgroup per slice,
// so that a few rows still spread over many CUs. Two kernels on one stream: k_split_reduce writes
// residual_out and each slice's square-sum into `partial`; k_split_norm sums a row's partials in
// slice order (the same bits in every workgroup of the row) and normalises its slice. The second
// launch is the combine; it needs no wait inside a kernel. Workgroup b of a launch handles slice
// b % splits of row b / splits, one pack per thread.
struct SplitArgs {
    RowArgs r;        // the buffers, eps and row length, as for k_rows
    float *partial;   // [rows, splits] square-sums of the slices: the caller's workspace
    int splits;       // slices per row
    int slice_packs;  // packs per slice (the last slice of a row may hold fewer)
};

template <int N, bool kStream>
__global__ void __launch_bounds__(1024) k_split_reduce(SplitArgs a)
{
    __shared__ float slots[kMaxWaves];
    const uint32_t splits = (uint32_t)a.splits;
    const uint32_t row = blockIdx.x / splits;
    const uint32_t slice = blockIdx.x - row * splits;
    const uint32_t packs = (uint32_t)a.r.packs;
    const uint32_t p = slice * (uint32_t)a.slice_packs + threadIdx.x;
    const size_t row_bytes = (size_t)row * packs * sizeof(u32x4);
    float ss = 0.0f;
    if (threadIdx.x < (uint32_t)a.slice_packs && p < packs) {
        const uint32_t off = p * (uint32_t)sizeof(u32x4);
        u32x4 x[N];
#pragma unroll
        for (int i = 0; i < N; ++i)
            x[i] = load_once<kStream>(reinterpret_cast<const char *>(a.r.in[i]) + row_bytes, off);
        const u32x4 res = load_once<kStream>(reinterpret_cast<const char *>(a.r.residual) + row_bytes, off);
        __builtin_amdgcn_sched_barrier(0);
        const u32x4 ro = add_residual<N>(x, res);
        // read straight back by k_split_norm: an ordinary store, so that it can stay in the caches
        store_pack(reinterpret_cast<char *>(a.r.residual_out) + row_bytes, off, ro);
        ss = add_squares(widen(ro), ss);
    }
    const float total = block_sum<false>(ss, slots);
    if (threadIdx.x == 0)
        a.partial[blockIdx.x] = total;
}

__global__ void __launch_bounds__(1024) k_split_norm(SplitArgs a)
{
    // this kernel's arguments in one scalar round trip (see args_in_sgprs)
    asm volatile("" ::"s"(a.partial), "s"(a.r.residual_out), "s"(a.r.weight), "s"(a.r.out),
                 "s"(a.splits), "s"(a.slice_packs), "s"(a.r.packs), "s"(blockDim.x));
    const uint32_t splits = (uint32_t)a.splits;
    const uint32_t row = blockIdx.x / splits;
    const uint32_t slice = blockIdx.x - row * splits;
    const uint32_t packs = (uint32_t)a.r.packs;
    const uint32_t p = slice * (uint32_t)a.slice_packs + threadIdx.x;
    const size_t row_bytes = (size_t)row * packs * sizeof(u32x4);
    const bool active = threadIdx.x < (uint32_t)a.slice_packs && p < packs;
    const uint32_t off = p * (uint32_t)sizeof(u32x4);
    // the slice's residual_out and weight do not depend on the row statistic: their loads go out
    // first, so that their round trip overlaps the one for the square-sums
    u32x4 yv = {0, 0, 0, 0}, gv = {0, 0, 0, 0};
    if (active) {
        yv = load_pack(reinterpret_cast<const char *>(a.r.residual_out) + row_bytes, off);
        gv = load_pack(reinterpret_cast<const char *>(a.r.weight), off);
    }
    // the row's slice square-sums (at most 64, and a workgroup is whole waves) are loaded at once,
    // lane i taking slice i, then added in slice order from registers: one memory round trip
    // instead of a load and a wait per slice
    const float *part = a.partial + (size_t)row * splits;
    const uint32_t lane = threadIdx.x & 63;
    const float mine = lane < splits ? part[lane] : 0.0f;
    float total = lane_value(mine, 0);
    for (uint32_t i = 1; i < splits; ++i)
        total = total + lane_value(mine, (int)i);
    float rstd = rsqrt_f32(total * a.r.inv_hidden + a.r.eps, a.r.tiny_eps);
    if (a.r.tiny_eps && total < kTinySquareSum) {
        // as in row_pass: the square-sum again at a 2^100 scale, here over the whole row's
        // residual_out (written by k_split_reduce), in the same order in every workgroup of the
        // row; a uniform branch, since every workgroup of the row holds the same total
        __shared__ float slots[kMaxWaves];
        const char *row_ro = reinterpret_cast<const char *>(a.r.residual_out) + row_bytes;
        float ss2 = 0.0f;
        for (uint32_t q = threadIdx.x; q < packs; q += blockDim.x) {
            const F8 y = widen(load_pack(row_ro, q * (uint32_t)sizeof(u32x4)));
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float z = y.v[e] * 0x1p100f;
                ss2 = __builtin_fmaf(z, z, ss2);
            }
        }
        const float total2 = block_sum<false>(ss2, slots);
        rstd = 0x1p100f * __builtin_amdgcn_rsqf(total2 * a.r.inv_hidden + a.r.eps * 0x1p100f * 0x1p100f);
    }
    if (active)
        store_stream(reinterpret_cast<char *>(a.r.out) + row_bytes, off,
                     normalise(widen(yv), widen(gv), rstd));
}

// Stage 1 with LDS staging, one wave per input (the one-wave-per-rank design that the flat reduce
// replaced: aiter PR #3817, Technical Details > 2stage > reduce-scatter), kept for comparison.
// The page describes it only as staging through LDS with a workgroup barrier, one wave per rank;
// this is a reading of that: a workgroup of N waves owns a tile of 64 * N packs; wave w copies
// input w's tile into LDS (N packs per lane), one barrier, then thread t reduces pack t of the
// tile over the N staged copies in input order and stores it. Bit-identical to k_flat_reduce.
template <int N, bool kStream>
__global__ void __launch_bounds__(64 * N) k_stage1_lds(FlatArgs a)
{
    __shared__ u32x4 tile[N][64 * N];
    // the wave index is uniform across the wave: reading it from lane 0 lets the compiler keep
    // the wave's input pointer in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const size_t first = (size_t)blockIdx.x * (64 * N);
    const char *src = reinterpret_cast<const char *>(a.in[wave]);
#pragma unroll
    for (int j = 0; j < N; ++j) {
        const int q = j * 64 + lane;
        if (first + q < a.packs)
            tile[wave][q] = load_once<kStream>(src + first * sizeof(u32x4), (uint32_t)q * sizeof(u32x4));
    }
    __syncthreads();
    const int t = threadIdx.x;
    if (first + t < a.packs) {
        u32x4 x[N];
#pragma unroll
        for (int i = 0; i < N; ++i)
            x[i] = tile[i][t];
        store_pack(reinterpret_cast<char *>(a.out) + first * sizeof(u32x4),
                   (uint32_t)t * sizeof(u32x4), narrow(reduce_packs<N>(x)));
    }
}

}  // namespace fa
