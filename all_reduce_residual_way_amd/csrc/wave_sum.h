// wave_sum.h - sum of one float per lane over a 64-lane wavefront with DPP, and over a workgroup
// with one LDS exchange. The RMSNorm square-sum reduction of both paths (aiter PR #3817,
// Technical Details > 1stage and > 2stage > stage-2 RMSNorm reduce: a DPP tree inside the wave).
//
// Inside each 16-lane row, every step adds a lane's value to a partner lane's value with the two
// lanes using each other as partners, so both compute the same sum (IEEE addition commutes) and
// every lane of the row ends with bit-identical partial sums; two row broadcasts then gather the
// four row sums in lane 63. The tree is fixed, so the result is the same on every run.
#pragma once

#include <hip/hip_runtime.h>

namespace fa {

// DPP lane-select controls (CDNA "data parallel primitives" encodings).
enum : int {
    kDppQuadXor1 = 0xB1,     // quad_perm [1,0,3,2]: lane i reads lane i ^ 1
    kDppQuadXor2 = 0x4E,     // quad_perm [2,3,0,1]: lane i reads lane i ^ 2
    kDppRowHalfMirror = 0x141, // lane i reads lane 7 - i within each group of 8
    kDppRowMirror = 0x140,   // lane i reads lane 15 - i within each row of 16
    kDppRowBcast15 = 0x142,  // lane 15 of each row is read by every lane of the next row
    kDppRowBcast31 = 0x143,  // lane 31 is read by every lane of rows 2 and 3
};

template <int kCtrl>
__device__ __forceinline__ float dpp_partner(float x)
{
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, 0xF, 0xF, false));
}

// The broadcast forms write only the rows in kRowMask; the other lanes read +0, so adding the
// result leaves them unchanged.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ float dpp_rows(float x)
{
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, kRowMask, 0xF, false));
}

__device__ __forceinline__ float lane_value(float x, int lane)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

// Sum over the 64 lanes; lane 63 ends with the result (the other lanes with partial sums).
__device__ __forceinline__ float wave_sum_dpp(float x)
{
    x = x + dpp_partner<kDppQuadXor1>(x);      // pairs
    x = x + dpp_partner<kDppQuadXor2>(x);      // quads
    x = x + dpp_partner<kDppRowHalfMirror>(x); // the two quads of each group of 8
    x = x + dpp_partner<kDppRowMirror>(x);     // the two halves of each 16-lane row
    // every lane of row k now holds that row's sum r_k; combine the rows in lane 63:
    x = x + dpp_rows<kDppRowBcast15, 0xA>(x);  // rows 1 and 3: r1 + r0, r3 + r2
    x = x + dpp_rows<kDppRowBcast31, 0xC>(x);  // row 3: (r3 + r2) + (r1 + r0)
    // IEEE addition commutes, so that is (r0 + r1) + (r2 + r3) bit for bit
    return x;
}

// The same sum by an XOR butterfly through the LDS crossbar (ds_bpermute_b32): the design the
// DPP tree replaced (aiter PR #3817, Technical Details > 1stage), kept for comparison. Partners
// at distance 1, 2, 4, 8 hold the same sums as the DPP steps above, and the last two steps add
// (row 0 + row 1) + (row 2 + row 3), so every lane ends with the bits lane 63 holds above.
__device__ __forceinline__ float wave_sum_bpermute(float x)
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int partner = __builtin_amdgcn_ds_bpermute((lane ^ d) << 2, __builtin_bit_cast(int, x));
        x = x + __builtin_bit_cast(float, partner);
    }
    return x;
}

template <bool kBpermute>
__device__ __forceinline__ float wave_sum(float x)
{
    if constexpr (kBpermute)
        return wave_sum_bpermute(x);
    else
        return wave_sum_dpp(x);
}

// Sum over the workgroup (blockDim.x a multiple of 64, at most 1024) of values that are >= +0
// (square-sums): wave sums (lane 63 writes its wave's), one barrier, then in every wave lane i
// takes wave i's sum (lanes past the last wave take +0, which leaves a sum unchanged) and the first
// four DPP steps above add lanes 0..15, so every wave computes the same fixed tree and gets the
// same bits. `slots` is LDS with room for one float per wave; all threads of the workgroup must
// call this.
template <bool kBpermute>
__device__ __forceinline__ float block_sum(float x, float *slots)
{
    const float w = wave_sum<kBpermute>(x);
    const int lane = threadIdx.x & 63;
    if (lane == 63)
        slots[threadIdx.x >> 6] = w;
    __syncthreads();
    const int waves = blockDim.x >> 6;
    float v = lane < waves ? slots[lane] : 0.0f;
    v = v + dpp_partner<kDppQuadXor1>(v);
    v = v + dpp_partner<kDppQuadXor2>(v);
    v = v + dpp_partner<kDppRowHalfMirror>(v);
    v = v + dpp_partner<kDppRowMirror>(v);
    return lane_value(v, 0);
}

}  // namespace fa
