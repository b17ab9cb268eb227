// bf16x8.h - the 16-byte "pack" of eight bf16 values that every kernel moves with one
// global_load_dwordx4 / global_store_dwordx4, and its conversions to and from eight floats.
//
// The pack is the per-thread unit of the flat reduce, in which every thread sums one pack over all
// the ranks' buffers (aiter PR #3817, Technical Details > 2stage > reduce-scatter); the page does
// not give its width, and 16 bytes is the widest single vector memory access on gfx950.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Eight floats in registers; element e of a pack is the low (even e) or high (odd e) half of
// dword e / 2, since the lower address holds the lower half on this little-endian machine.
struct F8 {
    float v[8];
};

// bf16 -> fp32 is exact: a bf16 pattern is the upper half of the binary32 pattern.
__device__ __forceinline__ F8 widen(u32x4 p)
{
    F8 f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f.v[2 * i] = __builtin_bit_cast(float, p[i] << 16);
        f.v[2 * i + 1] = __builtin_bit_cast(float, p[i] & 0xFFFF0000u);
    }
    return f;
}

// fp32 -> bf16, round to nearest even. On gfx950 the compiler lowers this conversion to
// v_cvt_pk_bf16_f32, two values per instruction, honouring the default round-to-nearest-even mode.
__device__ __forceinline__ uint32_t narrow2(float lo, float hi)
{
    f32x2 two = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(two, bf16x2));
}

__device__ __forceinline__ u32x4 narrow(const F8 &f)
{
    u32x4 p;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        p[i] = narrow2(f.v[2 * i], f.v[2 * i + 1]);
    return p;
}

__device__ __forceinline__ void add_into(F8 &acc, const F8 &x)
{
#pragma unroll
    for (int e = 0; e < 8; ++e)
        acc.v[e] = acc.v[e] + x.v[e];
}

}  // namespace fa
