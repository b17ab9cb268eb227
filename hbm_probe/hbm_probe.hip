// hbm_probe.hip - libhbm_probe.so: plain streaming kernels that measure what HBM delivers on this
// GPU for three traffic mixes, as the practical ceilings the fused kernel is compared with:
//   read  - one read stream (every 16-byte pack XOR-folded into a register; nothing is written
//           unless the fold hits a fixed 128-bit pattern, so the loads cannot be removed)
//   copy  - one read and one write stream
//   mix   - nine read streams and two write streams at the same offsets, the byte mix of the
//           one-stage kernel at N = 8 (eight partial sums and the residual in, residual_out and out
//           out), with no arithmetic beyond an XOR and an add per pack; mix_rw the same with 5 or 9
//           read and 1 or 2 write streams (the first stage of the two-stage path at N = 4 and 8
//           reads N + 1 streams and writes one).
//   reads / writes - the read streams of a mix alone (XOR-folded, nothing written) and its write
//           streams alone (a pattern derived from the pack index): timed back to back, the same
//           bytes as the mix with the reads and the writes in separate launches.
// Measurement infrastructure for the benchmark only; the fused path does not use it.
// All kernels are grid-stride loops guarded by the element count. `nt` selects the cache policy:
// bit 0 non-temporal loads, bit 1 non-temporal stores (3: the fused kernel's policy for HBM-cold
// data).
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr unsigned kBlock = 256;
constexpr int kMixReads = 9;
constexpr int kMixWrites = 2;

template <bool kNT>
__device__ __forceinline__ u32x4 load(const u32x4 *p)
{
    if constexpr (kNT)
        return __builtin_nontemporal_load(p);
    else
        return *p;
}

template <bool kNT>
__device__ __forceinline__ void store(u32x4 *p, u32x4 v)
{
    if constexpr (kNT)
        __builtin_nontemporal_store(v, p);
    else
        *p = v;
}

// kUnroll packs per thread per trip, kUnroll grid-strides apart, all loaded before they are folded.
template <bool kNT, int kUnroll>
__global__ void __launch_bounds__(kBlock) k_read(const u32x4 *__restrict__ src, size_t packs,
                                                 u32x4 *__restrict__ sink)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    u32x4 fold = {0u, 0u, 0u, 0u};
    for (; i + (kUnroll - 1) * stride < packs; i += kUnroll * stride) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            v[u] = load<kNT>(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            fold ^= v[u];
    }
    for (; i < packs; i += stride)
        fold ^= load<kNT>(src + i);
    if (fold.x == 0x9E3779B9u && fold.y == 0x7F4A7C15u && fold.z == 0x85EBCA6Bu &&
        fold.w == 0xC2B2AE35u)
        sink[0] = fold;
}

template <bool kNTL, bool kNTS>
__global__ void __launch_bounds__(kBlock) k_copy(const u32x4 *__restrict__ src,
                                                 u32x4 *__restrict__ dst, size_t packs)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < packs; i += stride)
        store<kNTS>(dst + i, load<kNTL>(src + i));
}

struct MixArgs {
    const u32x4 *in[kMixReads];
    u32x4 *out[kMixWrites];
    size_t packs;  // packs per stream
};

// out[0] = XOR of the R inputs, out[1] (when W == 2) = out[0] + in[0] (lane-wise 32-bit add).
template <int R, int W, bool kNTL, bool kNTS>
__global__ void __launch_bounds__(kBlock) k_mix(MixArgs a)
{
    static_assert(R >= 1 && R <= kMixReads && W >= 1 && W <= kMixWrites, "stream counts");
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < a.packs; i += stride) {
        u32x4 v[R];
#pragma unroll
        for (int k = 0; k < R; ++k)
            v[k] = load<kNTL>(a.in[k] + i);
        u32x4 x = v[0];
#pragma unroll
        for (int k = 1; k < R; ++k)
            x ^= v[k];
        store<kNTS>(a.out[0] + i, x);
        if constexpr (W == 2)
            store<kNTS>(a.out[1] + i, x + v[0]);
    }
}

// The R read streams of a mix alone: each pack XOR-folded into a register, written to `sink` only
// if the fold hits a fixed pattern (as k_read).
template <int R, bool kNTL>
__global__ void __launch_bounds__(kBlock) k_reads(MixArgs a, u32x4 *__restrict__ sink)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    u32x4 fold = {0u, 0u, 0u, 0u};
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < a.packs; i += stride) {
        u32x4 v[R];
#pragma unroll
        for (int k = 0; k < R; ++k)
            v[k] = load<kNTL>(a.in[k] + i);
#pragma unroll
        for (int k = 0; k < R; ++k)
            fold ^= v[k];
    }
    if (fold.x == 0x9E3779B9u && fold.y == 0x7F4A7C15u && fold.z == 0x85EBCA6Bu &&
        fold.w == 0xC2B2AE35u)
        sink[0] = fold;
}

// The W write streams of a mix alone: pack i of stream k holds {i, i >> 32, k, ~i}.
template <int W, bool kNTS>
__global__ void __launch_bounds__(kBlock) k_writes(MixArgs a)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < a.packs; i += stride) {
#pragma unroll
        for (int k = 0; k < W; ++k) {
            const u32x4 v = {(uint32_t)i, (uint32_t)(i >> 32), (uint32_t)k, ~(uint32_t)i};
            store<kNTS>(a.out[k] + i, v);
        }
    }
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int launched()
{
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? 0 : static_cast<int>(e);
}

template <int R, int W>
void launch_mix(const MixArgs &a, int nt, int grid, hipStream_t stream)
{
    const dim3 g(static_cast<unsigned>(grid)), b(kBlock);
    switch (nt) {
    case 0: hipLaunchKernelGGL((k_mix<R, W, false, false>), g, b, 0, stream, a); break;
    case 1: hipLaunchKernelGGL((k_mix<R, W, true, false>), g, b, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((k_mix<R, W, false, true>), g, b, 0, stream, a); break;
    default: hipLaunchKernelGGL((k_mix<R, W, true, true>), g, b, 0, stream, a); break;
    }
}

// The arguments of a mix of `reads` and `writes` streams, checked: -1 for a bad argument.
// Either side may be absent (reads == 0 with in == nullptr, or writes == 0 with out == nullptr) for
// the read-only and write-only kernels; the mixes need both.
int mix_args(const void *const *in, int reads, void *const *out, int writes, size_t packs, int nt,
             int grid, MixArgs *a)
{
    if ((in == nullptr && reads != 0) || (out == nullptr && writes != 0) || packs == 0 || grid < 1 ||
        grid > (1 << 20) || nt < 0 || nt > 3 || reads < 0 || reads > kMixReads || writes < 0 ||
        writes > kMixWrites || reads + writes == 0)
        return -1;
    *a = MixArgs{};
    for (int k = 0; k < reads; ++k) {
        if (in[k] == nullptr || !aligned16(in[k]))
            return -1;
        a->in[k] = static_cast<const u32x4 *>(in[k]);
    }
    for (int k = 0; k < writes; ++k) {
        if (out[k] == nullptr || !aligned16(out[k]))
            return -1;
        a->out[k] = static_cast<u32x4 *>(out[k]);
    }
    a->packs = packs;
    return 0;
}

}  // namespace

// Status: 0, -1 for a bad argument (null or misaligned pointer, zero packs, grid outside
// 1..2^20, nt outside 0..3, unroll not 1, 4 or 8) before any launch, or a positive hipError_t from
// the launch.
// Buffers are device memory of at least `packs` 16-byte packs each; `sink` holds one pack.

extern "C" int hbm_probe_read(const void *src, size_t packs, void *sink, int nt, int unroll,
                              int grid, hipStream_t stream)
{
    if (src == nullptr || sink == nullptr || !aligned16(src) || !aligned16(sink) || packs == 0 ||
        grid < 1 || grid > (1 << 20) || nt < 0 || nt > 3)
        return -1;
    const u32x4 *s = static_cast<const u32x4 *>(src);
    u32x4 *k = static_cast<u32x4 *>(sink);
    const dim3 g(static_cast<unsigned>(grid)), b(kBlock);
    switch ((nt & 1 ? 10 : 0) + unroll) {  // a read has no stores: bit 1 is ignored
    case 1: hipLaunchKernelGGL((k_read<false, 1>), g, b, 0, stream, s, packs, k); break;
    case 4: hipLaunchKernelGGL((k_read<false, 4>), g, b, 0, stream, s, packs, k); break;
    case 8: hipLaunchKernelGGL((k_read<false, 8>), g, b, 0, stream, s, packs, k); break;
    case 11: hipLaunchKernelGGL((k_read<true, 1>), g, b, 0, stream, s, packs, k); break;
    case 14: hipLaunchKernelGGL((k_read<true, 4>), g, b, 0, stream, s, packs, k); break;
    case 18: hipLaunchKernelGGL((k_read<true, 8>), g, b, 0, stream, s, packs, k); break;
    default: return -1;
    }
    return launched();
}

extern "C" int hbm_probe_copy(const void *src, void *dst, size_t packs, int nt, int grid,
                              hipStream_t stream)
{
    if (src == nullptr || dst == nullptr || !aligned16(src) || !aligned16(dst) || packs == 0 ||
        grid < 1 || grid > (1 << 20) || nt < 0 || nt > 3)
        return -1;
    const u32x4 *s = static_cast<const u32x4 *>(src);
    u32x4 *d = static_cast<u32x4 *>(dst);
    const dim3 g(static_cast<unsigned>(grid)), b(kBlock);
    switch (nt) {
    case 0: hipLaunchKernelGGL((k_copy<false, false>), g, b, 0, stream, s, d, packs); break;
    case 1: hipLaunchKernelGGL((k_copy<true, false>), g, b, 0, stream, s, d, packs); break;
    case 2: hipLaunchKernelGGL((k_copy<false, true>), g, b, 0, stream, s, d, packs); break;
    default: hipLaunchKernelGGL((k_copy<true, true>), g, b, 0, stream, s, d, packs); break;
    }
    return launched();
}

// `in`: host array of 9 device pointers, `out`: host array of 2, each stream `packs` packs long.
extern "C" int hbm_probe_mix(const void *const *in, void *const *out, size_t packs, int nt,
                             int grid, hipStream_t stream)
{
    MixArgs a;
    if (in == nullptr || out == nullptr || mix_args(in, kMixReads, out, kMixWrites, packs, nt, grid, &a) != 0)
        return -1;
    launch_mix<kMixReads, kMixWrites>(a, nt, grid, stream);
    return launched();
}

// `in`: host array of `reads` device pointers (5 or 9), `out`: host array of `writes` (1 or 2).
extern "C" int hbm_probe_mix_rw(const void *const *in, int reads, void *const *out, int writes,
                                size_t packs, int nt, int grid, hipStream_t stream)
{
    MixArgs a;
    if ((reads != 5 && reads != 9) || writes < 1 || mix_args(in, reads, out, writes, packs, nt, grid, &a) != 0)
        return -1;
    if (reads == 5)
        writes == 1 ? launch_mix<5, 1>(a, nt, grid, stream) : launch_mix<5, 2>(a, nt, grid, stream);
    else
        writes == 1 ? launch_mix<9, 1>(a, nt, grid, stream) : launch_mix<9, 2>(a, nt, grid, stream);
    return launched();
}

// The read streams of a mix alone: `in` is a host array of `reads` device pointers (5 or 9), each
// `packs` packs long; `sink` holds one pack. Only bit 0 of `nt` applies (there are no stores).
extern "C" int hbm_probe_reads(const void *const *in, int reads, size_t packs, void *sink, int nt,
                               int grid, hipStream_t stream)
{
    MixArgs a;
    if ((reads != 5 && reads != 9) || sink == nullptr || !aligned16(sink) ||
        mix_args(in, reads, nullptr, 0, packs, nt, grid, &a) != 0)
        return -1;
    u32x4 *k = static_cast<u32x4 *>(sink);
    const dim3 g(static_cast<unsigned>(grid)), b(kBlock);
    switch (reads * 2 + (nt & 1)) {
    case 10: hipLaunchKernelGGL((k_reads<5, false>), g, b, 0, stream, a, k); break;
    case 11: hipLaunchKernelGGL((k_reads<5, true>), g, b, 0, stream, a, k); break;
    case 18: hipLaunchKernelGGL((k_reads<9, false>), g, b, 0, stream, a, k); break;
    default: hipLaunchKernelGGL((k_reads<9, true>), g, b, 0, stream, a, k); break;
    }
    return launched();
}

// The write streams of a mix alone: `out` is a host array of `writes` device pointers (1 or 2),
// each `packs` packs long. Only bit 1 of `nt` applies (there are no loads).
extern "C" int hbm_probe_writes(void *const *out, int writes, size_t packs, int nt, int grid,
                                hipStream_t stream)
{
    MixArgs a;
    if (writes < 1 || mix_args(nullptr, 0, out, writes, packs, nt, grid, &a) != 0)
        return -1;
    const dim3 g(static_cast<unsigned>(grid)), b(kBlock);
    switch (writes * 2 + ((nt >> 1) & 1)) {
    case 2: hipLaunchKernelGGL((k_writes<1, false>), g, b, 0, stream, a); break;
    case 3: hipLaunchKernelGGL((k_writes<1, true>), g, b, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((k_writes<2, false>), g, b, 0, stream, a); break;
    default: hipLaunchKernelGGL((k_writes<2, true>), g, b, 0, stream, a); break;
    }
    return launched();
}
