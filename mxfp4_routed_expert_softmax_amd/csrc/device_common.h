// device_common.h -- small device helpers shared by the gfx950 kernels of the
// routed-expert MoE layer.  Internal to the HIP library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace k3 {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

// E8M0 scale byte s -> 2^(s-127) as fp32 (s = 0 gives the subnormal 2^-127).
__device__ __forceinline__ float e8m0_f32(uint32_t s)
{
    return __uint_as_float(s ? (s << 23) : 0x00400000u);
}

// Byte SEL of w holds two E2M1 codes (low nibble = even element); the gfx950
// scaled convert yields both as fp32, multiplied by the power-of-two scale.
template <int SEL>
__device__ __forceinline__ f32x2 fp4x2_scaled(uint32_t w, float scale)
{
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, SEL);
}

// acc += sum over the 8 codes of w (elements 0..7) times xs[0..7].
__device__ __forceinline__ float dot8_fp4(uint32_t w, float scale, const float* xs, float acc)
{
    f32x2 a = fp4x2_scaled<0>(w, scale);
    f32x2 b = fp4x2_scaled<1>(w, scale);
    f32x2 c = fp4x2_scaled<2>(w, scale);
    f32x2 d = fp4x2_scaled<3>(w, scale);
    acc = __builtin_fmaf(a.x, xs[0], acc);
    acc = __builtin_fmaf(a.y, xs[1], acc);
    acc = __builtin_fmaf(b.x, xs[2], acc);
    acc = __builtin_fmaf(b.y, xs[3], acc);
    acc = __builtin_fmaf(c.x, xs[4], acc);
    acc = __builtin_fmaf(c.y, xs[5], acc);
    acc = __builtin_fmaf(d.x, xs[6], acc);
    acc = __builtin_fmaf(d.y, xs[7], acc);
    return acc;
}

// acc += (one 32-element MX block: 16 code bytes in q, scale) . xs[0..31]
__device__ __forceinline__ float dot32_fp4(uint4 q, float scale, const float* xs, float acc)
{
    acc = dot8_fp4(q.x, scale, xs + 0, acc);
    acc = dot8_fp4(q.y, scale, xs + 8, acc);
    acc = dot8_fp4(q.z, scale, xs + 16, acc);
    acc = dot8_fp4(q.w, scale, xs + 24, acc);
    return acc;
}

// Overflow-free SiLU in fp32: z / (1 + e^-z) (e^-z -> inf gives -0 for very
// negative z, the correct limit).
__device__ __forceinline__ float silu_f32(float z)
{
    return z / (1.0f + expf(-z));
}

template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int m, int width = kWave)
{
    return __shfl_xor(v, m, width);
}

__device__ __forceinline__ uint4 ldg16(const uint8_t* p)
{
    return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ void load32f(const float* p, float* xs)
{
    const float4* q = reinterpret_cast<const float4*>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float4 v = q[i];
        xs[4 * i + 0] = v.x;
        xs[4 * i + 1] = v.y;
        xs[4 * i + 2] = v.z;
        xs[4 * i + 3] = v.w;
    }
}

}  // namespace k3
