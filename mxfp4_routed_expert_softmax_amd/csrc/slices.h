// slices.h -- an fp32 block of 32 values written as the sum of kSlices
// MX-FP8 (E4M3 codes, one E8M0 scale per slice) "slices", for the matrix-core
// fp32-activation path.  Internal to the HIP library.
//
// Slice n is the E4M3 rounding, under an E8M0 scale taken from the block
// maximum of what slices 0..n-1 left over, of that remainder; every remainder
// is formed exactly in fp32.  Codes below 8 are left in the remainder, so a
// slice's codes span at most five binades (the scaled matrix core sums
// products over a wider span inexactly).  Each slice still cuts the block
// maximum of the remainder by 2^-4 or more, so six slices reproduce the block
// to within 2^-24 of its maximum -- one fp32 rounding -- for blocks whose
// maximum is at least 2^-100 (smaller ones are carried to within an absolute
// 2^-124).
#pragma once
#include "device_common.h"
#include "kernels.h"

namespace k3 {

typedef short sl_v2s __attribute__((ext_vector_type(2)));

// xor-swizzle inside 32-lane halves
template <int M>
__device__ __forceinline__ float sl_xor(float v)
{
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), (M << 10) | 0x1F));
}

__device__ __forceinline__ float max32(float v)
{
    v = fmaxf(v, sl_xor<1>(v));
    v = fmaxf(v, sl_xor<2>(v));
    v = fmaxf(v, sl_xor<4>(v));
    v = fmaxf(v, sl_xor<8>(v));
    v = fmaxf(v, sl_xor<16>(v));
    return v;
}

// The 32 lanes of a half-wave hold one 32-value block, one value each; lane
// gets its E4M3 code of every slice and the (uniform) E8M0 scale bytes.
// Slice scale: 2^s with s = floor(log2 m) - 7 for the remainder's block
// maximum m (so m / 2^s lies in [128, 256), inside E4M3's range), s >= -127.
__device__ __forceinline__ void split_block(float v, uint32_t (&code)[kSlices], uint32_t (&sbyte)[kSlices])
{
    float r = v;
#pragma unroll
    for (int n = 0; n < kSlices; ++n) {
        const float m = max32(fabsf(r));
        const int ex = (int)(__float_as_uint(m) >> 23) - 127;  // floor(log2 m); -127 for 0 / subnormal
        const int s = max(ex - 7, -127);
        const float down = __uint_as_float((uint32_t)(127 - s) << 23);  // 2^-s, normal for s in [-127, 120]
        const sl_v2s zero = {0, 0};
        const sl_v2s enc = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(zero, r * down, 0.0f, 1.0f, false);
        // a code below 8 (E4M3 exponent field < 10) is dropped and left in
        // the remainder for the next slice: it would leave the slice's codes
        // spanning more binades than the matrix core sums exactly
        uint32_t c = (uint32_t)(uint16_t)enc.x & 0xffu;
        c = (c & 0x78u) >= 0x50u ? c : 0u;
        const f32x2 back = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c, 1.0f, false);
        r -= back.x * e8m0_f32((uint32_t)(s + 127));  // exact: the remainder needs no rounding
        code[n] = c;
        sbyte[n] = (uint32_t)(s + 127);
    }
}

// Write one block's slices: codes [kSlices][n] bytes, scales [kSlices][n/32].
__device__ __forceinline__ void store_block(int lane32, int blk, int n, uint8_t* codes, uint8_t* scales,
                                            const uint32_t (&code)[kSlices], const uint32_t (&sbyte)[kSlices])
{
    const int nb = n >> 5;
#pragma unroll
    for (int j = 0; j < kSlices; ++j) {
        codes[(size_t)j * n + 32 * blk + lane32] = (uint8_t)code[j];
        if (lane32 == 0) scales[(size_t)j * nb + blk] = (uint8_t)sbyte[j];
    }
}

}  // namespace k3
