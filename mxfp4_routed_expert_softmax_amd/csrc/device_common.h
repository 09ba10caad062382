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

// Overflow-free SiLU in fp32: z / (1 + e^-z) (e^-z -> inf gives -0 for very
// negative z, the correct limit).
__device__ __forceinline__ float silu_f32(float z)
{
    return z / (1.0f + expf(-z));
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

// ---- buffer loads -------------------------------------------------------
// Weight rows are read through a buffer resource on the block's (uniform)
// matrix base: one 32-bit lane offset serves every row (the row offset is a
// scalar), and a lane whose offset is >= 2^31 reads zeros without touching
// memory -- the lanes past the end of the reduction axis.
constexpr uint32_t kOff = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t weight_rsrc(const uint8_t* base)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, 0x7fffffff, 0x00020000);
}

__device__ __forceinline__ uint4 ld_codes(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, (int)soff, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// The same load marked non-temporal (cache policy bit NT): for weight rows
// that one launch reads exactly once (the small-batch GEMVs).  A one-pass
// stream of several hundred MB runs about 15% faster this way on MI355X, and
// it leaves what is reused between launches (the router matrix) in the
// caches.  The grouped GEMMs re-read their weight tiles from L2 across token
// passes and keep ld_codes.
__device__ __forceinline__ uint4 ld_stream(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, (int)soff, 2);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ uint32_t ld_scale(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_amdgcn_raw_buffer_load_b8(r, voff, (int)soff, 0);
}

// ---- direct global->LDS copies (gfx950 global_load_lds_dwordx4) ---------
// LDS byte address of a pointer into __shared__ memory (the low half of the
// flat address; the shared aperture is 4 GiB aligned)
__device__ __forceinline__ uint32_t lds_addr(const void* p)
{
    return (uint32_t)reinterpret_cast<uintptr_t>(p);
}

// One 16-byte-per-lane global->LDS copy from base + off (base wave-uniform,
// in SGPRs; off per lane); lane l lands at LDS address m0 + 16*l.  Written as
// assembly so that the compiler neither serialises the copies nor waits on
// them before LDS reads: completion is awaited explicitly (vm_wait)
// before a stage is read.  m0 is restored; one wait state separates its
// write from the copy.
__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* p)
{
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<const uint8_t*>(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ void dma16(const uint8_t* base, uint32_t off, uint32_t m0)
{
    base = uniform_ptr(base);
    m0 = __builtin_amdgcn_readfirstlane(m0);
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(off), "s"(base), "s"(m0)
        : "memory");
}

// Copy nbytes (a multiple of 1 KiB) of contiguous global memory to LDS dst:
// the block's copies of 1 KiB go round-robin to its four waves.
__device__ __forceinline__ void lds_copy(const uint8_t* src, uint32_t dst, int nbytes)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (int j = wave; 1024 * j < nbytes; j += 4)
        dma16(src + 1024 * j, 16u * (uint32_t)lane, dst + 1024u * (uint32_t)j);
}

// Wait until at most N vector-memory loads issued by this wave are still in
// flight (they complete in issue order).  vmcnt sits in bits [3:0] and
// [15:14] of the immediate; expcnt (7) and lgkmcnt (15) are left free.
template <int N>
__device__ __forceinline__ void vm_wait()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

}  // namespace k3
